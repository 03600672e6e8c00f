// Internal helpers shared by the host-side translation units of libencscore.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/encscore.h"

namespace es {

// Record a message for es_last_error() on this thread and return `code`.
es_status fail(es_status code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

}  // namespace es
