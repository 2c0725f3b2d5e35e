// dw_tune.hip -- per-geometry kernel selection (the MegEngine large-kernel
// depthwise article's automatic choice among algorithms), measured on the
// device the library runs on.
//
// Every pass has several kernel families, and more than one of them can run a
// given geometry (e.g. a 16-bit 31x31 layer on the matrix cores or on the
// vector units; a 3x3 layer with the row-walk, the specialised band or the
// generic band kernel).  The built-in rules pick one; the selection table
// below overrides them per (pass, dtype, geometry):
//  - dwconv2d_algo_candidates lists the families that can run a geometry;
//  - dwconv2d_set_algo records (or removes) a family for it;
//  - dwconv2d_tune_{fwd,bwd_input,bwd_weight} time every candidate on the
//    caller's tensors with HIP events on the caller's stream and record the
//    fastest.
// The table is process-wide and guarded by a mutex; compute calls read it
// (only when it is not empty) when they choose their kernel.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "dw_internal.hpp"
#include "dwconv.h"

namespace dw {
namespace {

struct Key {
    int v[15];  // pass, dtype, then the 13 geometry integers
    bool operator==(const Key &o) const { return std::memcmp(v, o.v, sizeof(v)) == 0; }
};

struct KeyHash {
    size_t operator()(const Key &k) const {
        uint64_t h = 1469598103934665603ull;  // FNV-1a over the integers
        for (int x : k.v) {
            h ^= static_cast<uint32_t>(x);
            h *= 1099511628211ull;
        }
        return static_cast<size_t>(h);
    }
};

std::mutex g_mu;
std::unordered_map<Key, int, KeyHash> g_table;
std::atomic<int> g_entries{0};

Key make_key(int pass, const Geo &g, int dtype) {
    Key k;
    const int v[15] = {pass, dtype, g.n, g.ic, g.ih, g.iw, g.oc, g.kh, g.kw, g.sh, g.sw, g.ph, g.pw, g.dh, g.dw};
    std::memcpy(k.v, v, sizeof(v));
    return k;
}

}  // namespace

int tuned_algo(int pass, const Geo &g, int dtype) {
    if (g_entries.load(std::memory_order_acquire) == 0) return -1;
    std::lock_guard<std::mutex> lk(g_mu);
    const auto it = g_table.find(make_key(pass, g, dtype));
    return it == g_table.end() ? -1 : it->second;
}

void set_tuned_algo(int pass, const Geo &g, int dtype, int algo) {
    std::lock_guard<std::mutex> lk(g_mu);
    const Key k = make_key(pass, g, dtype);
    if (algo < 0)
        g_table.erase(k);
    else
        g_table[k] = algo;
    g_entries.store(static_cast<int>(g_table.size()), std::memory_order_release);
}

}  // namespace dw
