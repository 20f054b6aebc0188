// dispatch.hpp -- host-side dispatch table (no HIP dependencies).
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

namespace iq4xs {

constexpr int64_t GEMV_MAX_M_TABLE = 4;

struct Band {
    int path = 0;
    int64_t mlo = 0, mhi = 0;
    int64_t nlo = -1, nhi = -1, klo = -1, khi = -1;   // inclusive ranges; -1 = any
};

struct Table {
    std::string arch;
    int cus = 0;                  // compute units the bands were measured on (0: any)
    std::vector<Band> bands;
};

const char *path_name(int p);
bool parse_table(const std::string &text, Table *out, std::string *err);
// First band matching (M, N, K); DEQ_BF16 bands only when allow_bf16, BF16X3
// bands only when allow_x3 (IQ4_XS weights).  0 = none.
int table_lookup(const Table &t, int64_t M, int64_t N, int64_t K, bool allow_bf16, bool allow_x3 = true);
// The table compiled into the library (dispatch_gfx950.txt).
const char *default_table_text();

}  // namespace iq4xs
