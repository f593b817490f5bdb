// Internal to libvimscan.so: the per-thread error record (vs_last_error)
// shared by the library's translation units. Not part of the C ABI.
#pragma once

__attribute__((visibility("hidden"))) int vs_internal_fail(int code, const char* msg);
__attribute__((visibility("hidden"))) void vs_internal_clear_error();
