// Refusal messages shared by the library's source files.
#pragma once

namespace pgqa_detail {
// Records a printf-style message for pgqa_last_error() on this thread and
// returns `code`.
__attribute__((visibility("hidden"), format(printf, 2, 3))) int fail(int code, const char *fmt, ...);
// Clears this thread's message (at the start of every entry point).
__attribute__((visibility("hidden"))) void clear_error();
// This thread's message ("" if none).
__attribute__((visibility("hidden"))) const char *error_text();
}  // namespace pgqa_detail
