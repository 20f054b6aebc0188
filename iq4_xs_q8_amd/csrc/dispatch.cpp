// dispatch.cpp -- the measured crossover table behind IQ4XS_PATH_AUTO.
//
// "V100TPS engine log" (agent-report.daedalus.work/V100TPS/engine.html), mmvq vs
// dequant+GEMM table: the measured crossover sat near M = 15 while the
// dispatcher's threshold was hard-coded at 8 and picked a path 26% slower at
// M = 12; adding a format to an eligibility list without a kernel behind it
// produced silent garbage.  So the bands here are data (measured on the
// device, see the calibration script), the table names the device it was
// measured on, and a malformed table is rejected as a whole.
#include <cctype>
#include <cstdlib>
#include <sstream>
#include <string>
#include <vector>

#include "dispatch.hpp"
#include "iq4xs.h"

namespace iq4xs {

const char *path_name(int p)
{
    switch (p) {
    case IQ4XS_PATH_AUTO: return "AUTO";
    case IQ4XS_PATH_GEMV: return "GEMV";
    case IQ4XS_PATH_MMQ: return "MMQ";
    case IQ4XS_PATH_DEQ_BF16: return "DEQ_BF16";
    case IQ4XS_PATH_BF16X3: return "BF16X3";
    default: return "?";
    }
}

static int path_from_name(const std::string &s)
{
    for (int p = IQ4XS_PATH_GEMV; p < IQ4XS_NUM_PATHS; p++)
        if (s == path_name(p))
            return p;
    return 0;
}

static bool parse_int(const std::string &s, int64_t *v, bool allow_star)
{
    if (allow_star && s == "*") {
        *v = -1;
        return true;
    }
    if (s.empty() || s.size() > 18)
        return false;
    for (char c : s)
        if (!std::isdigit((unsigned char)c))
            return false;
    *v = std::strtoll(s.c_str(), nullptr, 10);
    return true;
}

// "*" (any), "v" or "lo-hi" (inclusive)
static bool parse_range(const std::string &s, int64_t *lo, int64_t *hi)
{
    if (s == "*") {
        *lo = *hi = -1;
        return true;
    }
    const size_t dash = s.find('-');
    if (dash == std::string::npos)
        return parse_int(s, lo, false) && parse_int(s, hi, false) && *lo >= 1;
    return parse_int(s.substr(0, dash), lo, false) && parse_int(s.substr(dash + 1), hi, false) && *lo >= 1 &&
           *hi >= *lo;
}

bool parse_table(const std::string &text, Table *out, std::string *err)
{
    Table t;
    std::istringstream in(text);
    std::string line;
    int lineno = 0;
    while (std::getline(in, line)) {
        lineno++;
        const size_t hash = line.find('#');
        if (hash != std::string::npos)
            line.resize(hash);
        std::istringstream ls(line);
        std::vector<std::string> tok;
        for (std::string w; ls >> w;)
            tok.push_back(w);
        if (tok.empty())
            continue;
        if (tok[0] == "arch" && tok.size() == 2) {
            t.arch = tok[1];
        } else if (tok[0] == "cus" && tok.size() == 2) {
            // the bands were measured on a device with this many compute
            // units; a device with another count (e.g. a partitioned one)
            // does not use them
            int64_t c = 0;
            if (!parse_int(tok[1], &c, false) || c < 1 || c > 65536) {
                *err = "dispatch table line " + std::to_string(lineno) + ": bad compute-unit count";
                return false;
            }
            t.cus = (int)c;
        } else if (tok[0] == "band" && tok.size() == 6) {
            Band b;
            b.path = path_from_name(tok[1]);
            if (!b.path || !parse_int(tok[2], &b.mlo, false) || !parse_int(tok[3], &b.mhi, false) ||
                !parse_range(tok[4], &b.nlo, &b.nhi) || !parse_range(tok[5], &b.klo, &b.khi) || b.mlo < 1 ||
                b.mhi < b.mlo) {
                *err = "dispatch table line " + std::to_string(lineno) + ": bad band";
                return false;
            }
            if (b.path == IQ4XS_PATH_GEMV && b.mhi > GEMV_MAX_M_TABLE) {
                *err = "dispatch table line " + std::to_string(lineno) + ": GEMV band beyond M=4";
                return false;
            }
            t.bands.push_back(b);
        } else {
            *err = "dispatch table line " + std::to_string(lineno) + ": unknown entry";
            return false;
        }
    }
    if (t.arch.empty()) {
        *err = "dispatch table has no arch line";
        return false;
    }
    if (t.bands.empty()) {
        *err = "dispatch table has no bands";
        return false;
    }
    *out = t;
    return true;
}

int table_lookup(const Table &t, int64_t M, int64_t N, int64_t K, bool allow_bf16, bool allow_x3)
{
    for (const Band &b : t.bands) {
        if ((b.path == IQ4XS_PATH_DEQ_BF16 && !allow_bf16) || (b.path == IQ4XS_PATH_BF16X3 && !allow_x3))
            continue;
        if (M < b.mlo || M > b.mhi)
            continue;
        if (b.nlo >= 0 && (N < b.nlo || N > b.nhi))
            continue;
        if (b.klo >= 0 && (K < b.klo || K > b.khi))
            continue;
        return b.path;
    }
    return 0;
}

const char *default_table_text()
{
    static const char text[] =
#include "dispatch_table.inc"
        ;
    return text;
}

}  // namespace iq4xs
