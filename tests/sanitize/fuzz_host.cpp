// Host-side fuzz of libgdn's C ABI (gdn_varlen_meta, gdn_split_meta,
// gdn_chunk_fwd, gdn_state_summary, gdn_state_merge, gdn_state_merge_pieces,
// gdn_chunk_bwd) under AddressSanitizer and
// UndefinedBehaviorSanitizer: random descriptors, unit offsets (valid and
// broken), flags, modes, capacities and workspace sizes. Input pointers are
// fake non-null addresses that nothing may dereference; output arrays of the
// metadata call are exactly as large as the capacity passed, so a write past
// them is reported. Exit status 0 when every call returned and every status
// was one of the declared ones.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <vector>

#include "gdn.h"

void stub_set_workspace(const void* base, size_t bytes);

namespace {
std::mt19937_64 rng(20261203);
int pick(std::initializer_list<int> xs) {
    std::uniform_int_distribution<size_t> d(0, xs.size() - 1);
    return *(xs.begin() + d(rng));
}
int uni(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }

void* const FAKE = reinterpret_cast<void*>(uintptr_t(1) << 40);
long counts[6] = {0, 0, 0, 0, 0, 0};

void tally(gdn_status s) {
    if (s < GDN_OK || s > GDN_ERR_CAPACITY) {
        fprintf(stderr, "undeclared status %d\n", (int)s);
        exit(2);
    }
    counts[s]++;
}

// offsets: mostly valid (0 < ... < total), sometimes broken
std::vector<int32_t> offsets(int64_t total, int n_units) {
    std::vector<int32_t> o(n_units + 1);
    o[0] = 0;
    for (int i = 1; i < n_units; ++i) o[i] = total > 0 ? (int32_t)uni(0, (int)std::min<int64_t>(total, 1 << 20)) : 0;
    o[n_units] = (int32_t)std::min<int64_t>(total, INT32_MAX);
    std::sort(o.begin() + 1, o.end() - 1);
    switch (uni(0, 9)) {
        case 0: if (n_units > 1) o[1] = o[0]; break;                    // empty unit
        case 1: o[0] = 1; break;                                        // does not start at 0
        case 2: o[n_units] += 1; break;                                 // does not end at the total
        case 3: if (n_units > 1) std::swap(o[0], o[n_units]); break;    // decreasing
        default: break;
    }
    return o;
}

void fuzz_meta() {
    const int n = uni(0, 40);
    std::vector<int32_t> o = offsets(uni(0, 5000), std::max(n - 1, 1));
    o.resize(n);
    const int32_t total = n ? o.back() : 0;
    int32_t cnt = -1;
    tally(gdn_varlen_meta(n ? o.data() : nullptr, n, total, pick({64, 0, -1, 1, 7}), nullptr, 0, nullptr, &cnt));
    const int cap = uni(0, 200);
    std::vector<int32_t> ci(2 * (size_t)cap + 1), co((size_t)std::max(n, 1));
    tally(gdn_varlen_meta(n ? o.data() : nullptr, n, total, 64, cap ? ci.data() : nullptr, cap,
                          n ? co.data() : nullptr, &cnt));
}

void fuzz_fwd() {
    gdn_desc d;
    memset(&d, 0, sizeof(d));
    d.B = pick({1, 1, 2, 3, 0, -1});
    d.T = pick({0, 1, 63, 64, 65, 200, 1000, 4096, 16384, 16400, -5});   // long rows: the pieced forward
    d.H = pick({1, 3, 16, 40, 0});
    d.K = pick({128, 128, 128, 64});
    d.V = pick({128, 128, 128, 64});
    d.layout = pick({0, 0, 1, 2});
    d.dtype = pick({0, 1, 1, 3});
    d.o_dtype = pick({0, 1, 2});
    d.gate_kind = pick({0, 1, 1, 5});
    d.use_exp2 = pick({0, 1, 4});
    d.chunk_size = pick({64, 64, 64, 32});
    d.scale = pick({0, 0, 1, 2}) == 2 ? __builtin_nanf("") : 0.0884f;
    std::vector<int32_t> o;
    if (d.layout == 1 || uni(0, 2) == 0) {
        const int64_t total = int64_t(std::max(d.B, 0)) * std::max(d.T, 0);
        const int n_units = uni(1, 30);
        o = offsets(total, n_units);
        // BSND segments must include every row start
        if (d.layout == 0 && d.B > 1 && uni(0, 1)) {
            o.clear();
            for (int b = 0; b < d.B; ++b) {
                o.push_back(b * d.T);
                if (d.T > 2) o.push_back(b * d.T + d.T / 2);
            }
            o.push_back(d.B * d.T);
        }
        d.n_units = (int32_t)o.size() - 1;
        d.offsets_host = o.data();
        d.offsets_dev = static_cast<const int32_t*>(uni(0, 9) ? FAKE : nullptr);
        d.chunk_offsets_dev = static_cast<const int32_t*>(FAKE);
        d.chunk_indices_dev = static_cast<const int32_t*>(FAKE);
    }
    size_t need = 0;
    gdn_status s = gdn_chunk_fwd(&d, FAKE, FAKE, FAKE, (const float*)FAKE, FAKE, nullptr, FAKE, nullptr,
                                 nullptr, 0, nullptr, &need, nullptr);
    tally(s);
    if (s != GDN_OK || need > (size_t(64) << 20)) return;
    const size_t have = uni(0, 4) ? need : need - 1;
    void* ws = aligned_alloc(256, (have + 255) / 256 * 256 + 256);
    stub_set_workspace(ws, have);
    size_t nb = have;
    const int flags = pick({0, 0, 1, 2, 3, 4, 8, 12, 16});
    void* q = uni(0, 9) ? FAKE : nullptr;
    tally(gdn_chunk_fwd(&d, q, FAKE, FAKE, (const float*)FAKE, FAKE, nullptr, FAKE, nullptr, nullptr, flags,
                        uni(0, 9) ? ws : static_cast<char*>(ws) + 64, &nb, nullptr));
    nb = have;
    const int mode = pick({0, 1, 2, 3});
    const int n_sel = pick({-1, -1, 0, 1, 3, 40});
    tally(gdn_state_summary(&d, q, FAKE, FAKE, (const float*)FAKE, FAKE, mode, pick({0, 0, 1, 2}),
                            uni(0, 5) ? static_cast<const int32_t*>(FAKE) : nullptr, n_sel, (float*)FAKE,
                            uni(0, 5) ? (float*)FAKE : nullptr, ws, &nb, nullptr));
    stub_set_workspace(nullptr, 0);
    free(ws);
    // the backward, with its own (larger) workspace
    size_t bneed = 0;
    void* p15[15];
    for (int i = 0; i < 15; ++i) p15[i] = uni(0, 19) ? FAKE : nullptr;
    const int bflags = pick({0, 0, 1, 2});
    s = gdn_chunk_bwd(&d, p15[0], p15[1], p15[2], (const float*)p15[3], p15[4], (const float*)p15[5], p15[6],
                      (const float*)p15[7], (float*)p15[8], (float*)p15[9], (float*)p15[10], (float*)p15[11],
                      (float*)p15[12], (float*)p15[13], bflags, nullptr, &bneed, nullptr);
    tally(s);
    if (s != GDN_OK || bneed > (size_t(128) << 20)) return;
    const size_t bhave = uni(0, 4) ? bneed : bneed - 256;
    void* bws = aligned_alloc(256, (bhave + 255) / 256 * 256 + 256);
    stub_set_workspace(bws, bhave);
    size_t bnb = bhave;
    tally(gdn_chunk_bwd(&d, p15[0], p15[1], p15[2], (const float*)p15[3], p15[4], (const float*)p15[5], p15[6],
                        (const float*)p15[7], (float*)p15[8], (float*)p15[9], (float*)p15[10], (float*)p15[11],
                        (float*)p15[12], (float*)p15[13], bflags, bws, &bnb, nullptr));
    bnb = bhave;
    stub_set_workspace(bws, bhave);
    tally(gdn_state_grad_summary(&d, p15[0], p15[1], p15[2], (const float*)p15[3], p15[4], (const float*)p15[5],
                                 p15[6], (float*)p15[13], bflags, bws, &bnb, nullptr));
    stub_set_workspace(nullptr, 0);
    free(bws);
}

// pieces of random documents cut by random segments; the pieces written must
// tile the token range, and a too-small capacity must write nothing past it
void fuzz_split_meta() {
    const int total = uni(1, 3000);
    std::vector<int32_t> docs = offsets(total, uni(1, 20)), segs = offsets(total, uni(1, 9));
    int32_t n = -1;
    const gdn_status s0 = gdn_split_meta(docs.data(), (int32_t)docs.size(), segs.data(), (int32_t)segs.size(), total,
                                         nullptr, nullptr, nullptr, 0, &n);
    tally(s0);
    if (s0 != GDN_OK) return;
    const int cap = uni(0, 2) ? n : uni(0, n);
    std::vector<int32_t> po((size_t)cap + 1), pd((size_t)std::max(cap, 1)), ps((size_t)std::max(cap, 1));
    const gdn_status s1 = gdn_split_meta(docs.data(), (int32_t)docs.size(), segs.data(), (int32_t)segs.size(), total,
                                         po.data(), pd.data(), ps.data(), cap, &n);
    tally(s1);
    if (s1 != GDN_OK) return;
    if (po[0] != 0 || po[n] != total) exit(4);
    for (int i = 0; i < n; ++i)
        if (po[i] >= po[i + 1] || (i && (pd[i] < pd[i - 1] || ps[i] < ps[i - 1]))) exit(4);
}

void fuzz_merge() {
    tally(gdn_state_merge_adjoint(pick({1, 2, 0}), pick({1, 8, 0}), pick({0, 1, 8, -1}), pick({128, 64}), 128,
                                  (const float*)FAKE, uni(0, 5) ? (const float*)FAKE : nullptr, nullptr, (float*)FAKE,
                                  nullptr, nullptr));
    tally(gdn_state_merge_pieces(pick({0, 1, 9, -1}), pick({1, 3, 0}), pick({1, 8, 0}), pick({128, 64}), 128,
                                 static_cast<const int32_t*>(uni(0, 5) ? FAKE : nullptr), (const float*)FAKE,
                                 (const float*)FAKE, nullptr, (float*)FAKE, nullptr));
    tally(gdn_state_merge(pick({1, 2, 0}), pick({1, 8, 0}), pick({0, 1, 8, -1}), pick({128, 64}), 128,
                          (const float*)FAKE, uni(0, 5) ? (const float*)FAKE : nullptr, nullptr, (float*)FAKE,
                          nullptr, nullptr));
}
}  // namespace

int main() {
    for (int i = 0; i < 4000; ++i) {
        fuzz_meta();
        fuzz_fwd();
        fuzz_merge();
        fuzz_split_meta();
    }
    printf("statuses: ok %ld invalid %ld unsupported %ld device %ld capacity %ld\n", counts[0], counts[1],
           counts[2], counts[3], counts[4]);
    return (counts[0] > 0 && counts[1] > 0 && counts[4] > 0) ? 0 : 3;
}
