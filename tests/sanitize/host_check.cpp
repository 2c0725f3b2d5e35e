// host_check.cpp -- drives every host-side path of the C ABI in include/dwconv.h
// (argument validation, output sizes, kernel-family selection and its table,
// workspace sizing, status strings) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Built from the library's sources compiled for
// the host only, so no kernel is ever launched: every compute call below is
// one that validation rejects before any HIP call, and every pointer is a
// fake address that is never dereferenced.  Exit status 0 when every check
// holds; the sanitizers abort on the first finding.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <set>
#include <string>

#include "dwconv.h"

namespace {

int g_fail = 0;

#define CHECK(cond)                                                       \
    do {                                                                  \
        if (!(cond)) {                                                    \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++g_fail;                                                     \
        }                                                                 \
    } while (0)

void *fake(uint64_t off) { return reinterpret_cast<void *>((uint64_t{1} << 40) + off); }

struct Geo {
    int64_t v[13];
};

Geo geo(int64_t n = 2, int64_t ic = 3, int64_t ih = 9, int64_t iw = 7, int64_t oc = 3, int64_t kh = 3,
        int64_t kw = 3, int64_t sh = 1, int64_t sw = 1, int64_t ph = 1, int64_t pw = 1, int64_t dh = 1,
        int64_t dw = 1) {
    return Geo{{n, ic, ih, iw, oc, kh, kw, sh, sw, ph, pw, dh, dw}};
}

#define G(g) g.v[0], g.v[1], g.v[2], g.v[3], g.v[4], g.v[5], g.v[6], g.v[7], g.v[8], g.v[9], g.v[10], g.v[11], g.v[12]

// deterministic 64-bit LCG (Knuth's MMIX constants)
uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next() {
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return g_state >> 11;
}
int64_t pick(int64_t lo, int64_t hi) { return lo + static_cast<int64_t>(next() % static_cast<uint64_t>(hi - lo + 1)); }

void validation() {
    const Geo g = geo();
    CHECK(dwconv2d_fwd(fake(0), fake(0), nullptr, fake(4096), G(g), 7, nullptr) == DW_EDTYPE);
    CHECK(dwconv2d_fwd(nullptr, fake(0), nullptr, fake(4096), G(g), 0, nullptr) == DW_EPTR);
    CHECK(dwconv2d_fwd(fake(2), fake(0), nullptr, fake(4096), G(g), 0, nullptr) == DW_EPTR);
    CHECK(dwconv2d_fwd(fake(0), fake(0), nullptr, fake(0), G(g), 0, nullptr) == DW_EALIAS);
    CHECK(dwconv2d_fwd(fake(0), fake(4096), fake(8), fake(4088), G(g), 0, nullptr) == DW_EALIAS);
    const Geo m4 = geo(2, 3, 9, 7, 4);
    CHECK(dwconv2d_fwd(fake(0), fake(0), nullptr, fake(4096), G(m4), 0, nullptr) == DW_EMULT);
    CHECK(dwconv2d_bwd_input(fake(0), fake(0), fake(0), G(g), 0, nullptr) == DW_EALIAS);
    CHECK(dwconv2d_bwd_input(fake(0), fake(0), fake(4096), G(g), 3, nullptr) == DW_EDTYPE);
    size_t need = 0;
    CHECK(dwconv2d_bwd_weight_workspace_bytes(G(g), 0, &need) == DW_OK && need > 0);
    CHECK(dwconv2d_bwd_weight(fake(0), fake(0), fake(8192), nullptr, fake(1 << 20), need - 1, G(g), 0, nullptr) ==
          DW_EWORKSPACE);
    CHECK(dwconv2d_bwd_weight(fake(0), fake(0), fake(8192), nullptr, fake((1 << 20) + 4), need, G(g), 0,
                              nullptr) == DW_EWORKSPACE);
    CHECK(dwconv2d_bwd_weight(fake(0), fake(0), fake(8192), nullptr, fake(0), need, G(g), 0, nullptr) ==
          DW_EALIAS);
    CHECK(dwconv2d_bwd_weight_noalloc(fake(0), fake(0), fake(0), nullptr, G(g), 0, nullptr) == DW_EALIAS);
    const Geo big = geo(1, 2048, 8, 8, 16384, 31, 31, 1, 1, 15, 15);
    CHECK(dwconv2d_bwd_weight_noalloc(fake(0), fake(1 << 29), fake(1ull << 30), nullptr, G(big), 0, nullptr) ==
          DW_ESCRATCH);

    const void *f3[3] = {fake(1 << 24), fake(2 << 24), fake(3 << 24)};
    const int32_t d3[3] = {1, 3, 5};
    const int32_t bad[3] = {1, 0, 5};
    CHECK(dynconv_multidil_fwd(fake(0), f3, d3, 3, fake(8 << 24), 1, 4, 8, 8, 4, 0, nullptr) == DW_EDYN);
    CHECK(dynconv_multidil_fwd(fake(0), f3, bad, 3, fake(8 << 24), 1, 4, 8, 8, 3, 0, nullptr) == DW_EDYN);
    CHECK(dynconv_multidil_fwd(fake(0), f3, d3, 5, fake(8 << 24), 1, 4, 8, 8, 3, 0, nullptr) == DW_EDYN);
    CHECK(dynconv_multidil_fwd(fake(0), f3, d3, 3, fake(1 << 24), 1, 4, 8, 8, 3, 0, nullptr) == DW_EALIAS);
    CHECK(dynconv_multidil_fwd_into(fake(0), f3, d3, 3, fake(8 << 24), 12, 1, 1, 4, 8, 8, 3, 0, nullptr) ==
          DW_ESHAPE);
    void *g3[3] = {fake(10 << 24), fake((10 << 24) + 64), fake(12 << 24)};
    CHECK(dynconv_multidil_bwd(fake(0), f3, fake(8 << 24), d3, 3, fake(9 << 24), g3, 1, 4, 8, 8, 3, 0, nullptr) ==
          DW_EALIAS);
    CHECK(dynconv_multidil_bwd(fake(0), f3, fake(8 << 24), d3, 3, nullptr, nullptr, 1, 4, 8, 8, 3, 0, nullptr) ==
          DW_OK);  // nothing requested: validated, nothing launched
    CHECK(dynconv_multidil_bwd_from(fake(0), f3, fake(8 << 24), 12, 1, d3, 3, fake(9 << 24), nullptr, 1, 4, 8, 8,
                                    3, 0, nullptr) == DW_ESHAPE);

    // tuning entry points validate exactly like the compute calls
    CHECK(dwconv2d_tune_fwd(fake(0), fake(0), nullptr, fake(0), G(g), 0, 3, nullptr, nullptr) == DW_EALIAS);
    CHECK(dwconv2d_tune_bwd_input(fake(0), fake(0), fake(4096), G(g), 9, 3, nullptr, nullptr) == DW_EDTYPE);
    CHECK(dwconv2d_tune_bwd_weight(fake(0), fake(0), fake(8192), nullptr, nullptr, 0, G(g), 0, 3, nullptr,
                                   nullptr) == DW_EWORKSPACE);

    for (int s = -20; s <= 5; ++s) CHECK(dw_status_str(s) != nullptr && strlen(dw_status_str(s)) > 0);
}

// Every valid geometry gets a family for every pass and dtype, the family is
// among the candidates, and the workspace query agrees with the output size.
void selection(int count) {
    const char *names[64];
    for (int it = 0; it < count; ++it) {
        Geo g;
        const int64_t ic = pick(1, 300), mult = (next() % 4 == 0) ? pick(2, 4) : 1;
        const int64_t kh = (next() % 3 == 0) ? 31 : pick(1, 13), kw = (next() % 4 == 0) ? pick(1, 13) : kh;
        const bool wide = next() % 8 == 0;
        g = geo(pick(1, 130), ic, pick(1, wide ? 40 : 150), wide ? pick(1000, 40000) : pick(1, 150), ic * mult, kh,
                kw, pick(1, 3), pick(1, 3), pick(0, 16), pick(0, 16), pick(1, 3), pick(1, 3));
        if (next() % 16 == 0) g.v[4] = ic * mult + 1;  // not a multiple
        if (next() % 32 == 0) g.v[0] = int64_t{1} << 31;  // too large
        int64_t oh = -1, ow = -1;
        const int rc = dwconv2d_out_size(G(g), &oh, &ow);
        for (int dt = 0; dt < 3; ++dt) {
            size_t ws = 0;
            const int wrc = dwconv2d_bwd_weight_workspace_bytes(G(g), dt, &ws);
            CHECK(wrc == rc);
            for (int pass = 0; pass < 3; ++pass) {
                const char *a = dwconv2d_algo(pass, G(g), dt);
                CHECK((a != nullptr) == (rc == DW_OK));
                const int nc = dwconv2d_algo_candidates(pass, G(g), dt, names, 64);
                if (rc != DW_OK) {
                    CHECK(nc == rc);
                    continue;
                }
                CHECK(nc >= 1 && nc <= 64 && ws > 0 && oh >= 1 && ow >= 1);
                bool found = false;
                for (int i = 0; i < nc && i < 64; ++i) found = found || strcmp(names[i], a) == 0;
                CHECK(found);
            }
        }
    }
}

// The selection table: entries for many keys, overrides, removal.
void table() {
    const char *names[64];
    std::set<std::string> seen;
    for (int it = 0; it < 400; ++it) {
        const int64_t c = pick(1, 64);
        const Geo g = geo(pick(1, 8), c, pick(3, 70), pick(3, 70), c, 3, 3, pick(1, 2), pick(1, 2), 1, 1, 1, 1);
        const int pass = it % 3, dt = (it / 3) % 3;
        const char *base = dwconv2d_algo(pass, G(g), dt);
        const int nc = dwconv2d_algo_candidates(pass, G(g), dt, names, 64);
        CHECK(base != nullptr && nc >= 1);
        const char *pickn = names[next() % static_cast<uint64_t>(nc < 64 ? nc : 64)];
        CHECK(dwconv2d_set_algo(pass, G(g), dt, pickn) == DW_OK);
        CHECK(strcmp(dwconv2d_algo(pass, G(g), dt), pickn) == 0);
        std::string copy(pickn);  // the table must not keep our buffer
        char buf[64];
        snprintf(buf, sizeof(buf), "%s", copy.c_str());
        CHECK(dwconv2d_set_algo(pass, G(g), dt, buf) == DW_OK);
        memset(buf, 'x', sizeof(buf) - 1);
        CHECK(strcmp(dwconv2d_algo(pass, G(g), dt), copy.c_str()) == 0);
        CHECK(dwconv2d_set_algo(pass, G(g), dt, "no_such_family") != DW_OK);
        if (it % 2 == 0) {
            CHECK(dwconv2d_set_algo(pass, G(g), dt, nullptr) == DW_OK);
            CHECK(strcmp(dwconv2d_algo(pass, G(g), dt), base) == 0);
        }
        seen.insert(copy);
    }
    CHECK(!seen.empty());
}

}  // namespace

int main() {
    validation();
    selection(3000);
    table();
    if (g_fail) {
        fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    printf("host checks ok\n");
    return 0;
}
