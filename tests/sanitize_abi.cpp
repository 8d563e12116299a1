// Host-side checks of libattn's C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
// (host code only; no device code is compiled into this program and no GPU is touched).
//
// Every call made here fails the library's host-side validation or is an empty problem, so none of
// them reaches a HIP call: the fake device pointers are never dereferenced.  The sanitizers watch the
// validation itself (size products near INT_MAX, pointer-range arithmetic for the overlap checks,
// status strings), and each call's status is compared with the one the header documents.
//
// Exit status 0 when every status matched; the sanitizers abort the program on any finding.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <functional>
#include <limits>
#include <string>
#include <vector>

#include "attn.h"

namespace {

int g_fail = 0, g_calls = 0;

void expect(const std::string &what, int got, int want)
{
    ++g_calls;
    if (got != want) {
        ++g_fail;
        std::fprintf(stderr, "MISMATCH %s: status %d (%s), expected %d\n", what.c_str(), got,
                     attn_status_string(got), want);
    }
}

// Distinct, 16-byte aligned, never dereferenced addresses 64 GiB apart.
void *fake(int i) { return reinterpret_cast<void *>(uintptr_t(0x7f0000000000ULL) + (uintptr_t(i) << 36)); }

struct Sizes {
    int B = 1, H = 2, Hk = 1, Nq = 64, Nk = 80, d = 128, causal = 0;
    float scale = 0.125f;
    int ns = 4;
    long long wsb = -1;  // -1: exactly the workspace the call needs
};

// One entry point: how many pointer arguments it takes, which of them are outputs, its 16-byte alignment
// rule (the per-head scale arrays of the 8-bit forward only need 4), and a call through it.
struct Entry {
    const char *name;
    int nptr;
    std::vector<int> outputs;
    std::vector<int> align4;
    bool one_length;      // takes H and N (Hk = H, Nq = Nk = N)
    bool has_causal;
    bool has_scale;
    bool has_splits;
    std::function<int(void **, const Sizes &)> call;
};

std::vector<Entry> entries()
{
    std::vector<Entry> e;
    e.push_back({"attn_fwd", 5, {3, 4}, {}, true, true, true, false, [](void **p, const Sizes &s) {
                     return attn_fwd(p[0], p[1], p[2], p[3], (float *)p[4], s.B, s.H, s.Nq, s.d, s.causal, s.scale,
                                     nullptr);
                 }});
    e.push_back({"attn_fwd_qk", 5, {3, 4}, {}, false, true, true, false, [](void **p, const Sizes &s) {
                     return attn_fwd_qk(p[0], p[1], p[2], p[3], (float *)p[4], s.B, s.H, s.Hk, s.Nq, s.Nk, s.d,
                                        s.causal, s.scale, nullptr);
                 }});
    e.push_back({"attn_fwd_splitkv", 6, {3, 4, 5}, {}, false, true, true, true, [](void **p, const Sizes &s) {
                     long long wsb = s.wsb >= 0 ? s.wsb : attn_fwd_splitkv_workspace_size(s.B, s.H, s.Nq, s.d, s.ns);
                     if (wsb < 0) wsb = 0;
                     return attn_fwd_splitkv(p[0], p[1], p[2], p[3], (float *)p[4], s.B, s.H, s.Hk, s.Nq, s.Nk, s.d,
                                             s.causal, s.scale, s.ns, p[5], wsb, nullptr);
                 }});
    e.push_back({"attn_fwd_splitkv_noalloc", 5, {3, 4}, {}, false, true, true, true, [](void **p, const Sizes &s) {
                     return attn_fwd_splitkv_noalloc(p[0], p[1], p[2], p[3], (float *)p[4], s.B, s.H, s.Hk, s.Nq,
                                                     s.Nk, s.d, s.causal, s.scale, s.ns, nullptr);
                 }});
    e.push_back({"attn_fwd_fp8", 8, {6, 7}, {3, 4, 5}, false, true, true, false, [](void **p, const Sizes &s) {
                     return attn_fwd_fp8(p[0], p[1], p[2], (const float *)p[3], (const float *)p[4],
                                         (const float *)p[5], p[6], (float *)p[7], s.B, s.H, s.Hk, s.Nq, s.Nk, s.d,
                                         s.causal, s.scale, nullptr);
                 }});
    e.push_back({"attn_bwd", 10, {6, 7, 8, 9}, {}, true, true, true, false, [](void **p, const Sizes &s) {
                     return attn_bwd(p[0], p[1], p[2], p[3], p[4], (const float *)p[5], p[6], p[7], p[8],
                                     (float *)p[9], s.B, s.H, s.Nq, s.d, s.causal, s.scale, nullptr);
                 }});
    e.push_back({"attn_bwd_qk", 10, {6, 7, 8, 9}, {}, false, true, true, false, [](void **p, const Sizes &s) {
                     return attn_bwd_qk(p[0], p[1], p[2], p[3], p[4], (const float *)p[5], p[6], p[7], p[8],
                                        (float *)p[9], s.B, s.H, s.Hk, s.Nq, s.Nk, s.d, s.causal, s.scale, nullptr);
                 }});
    e.push_back({"attn_bwd_preprocess", 3, {2}, {}, true, false, false, false, [](void **p, const Sizes &s) {
                     return attn_bwd_preprocess(p[0], p[1], (float *)p[2], s.B, s.H, s.Nq, s.d, nullptr);
                 }});
    e.push_back({"attn_bwd_dkdv", 8, {6, 7}, {}, true, true, true, false, [](void **p, const Sizes &s) {
                     return attn_bwd_dkdv(p[0], p[1], p[2], p[3], (const float *)p[4], (const float *)p[5], p[6], p[7],
                                          s.B, s.H, s.Nq, s.d, s.causal, s.scale, nullptr);
                 }});
    e.push_back({"attn_bwd_dq", 7, {6}, {}, true, true, true, false, [](void **p, const Sizes &s) {
                     return attn_bwd_dq(p[0], p[1], p[2], p[3], (const float *)p[4], (const float *)p[5], p[6], s.B,
                                        s.H, s.Nq, s.d, s.causal, s.scale, nullptr);
                 }});
    e.push_back({"attn_bwd_dq_delta", 8, {6, 7}, {}, true, true, true, false, [](void **p, const Sizes &s) {
                     return attn_bwd_dq_delta(p[0], p[1], p[2], p[3], p[4], (const float *)p[5], (float *)p[6], p[7],
                                              s.B, s.H, s.Nq, s.d, s.causal, s.scale, nullptr);
                 }});
    return e;
}

Sizes base_sizes(const Entry &e)
{
    Sizes s;
    if (e.one_length) {
        s.H = 2;
        s.Hk = 2;
        s.Nq = s.Nk = 64;
    }
    return s;
}

void fill(void **p, int n)
{
    for (int i = 0; i < n; ++i) p[i] = fake(i);
}

void check_entry(const Entry &e)
{
    const std::string n = e.name;
    void *p[10];
    const Sizes s0 = base_sizes(e);

    // pointers: each one NULL, each one misaligned
    for (int i = 0; i < e.nptr; ++i) {
        fill(p, e.nptr);
        p[i] = nullptr;
        expect(n + " null arg " + std::to_string(i), e.call(p, s0), ATTN_ERR_NULLPTR);
        fill(p, e.nptr);
        const bool four = std::find(e.align4.begin(), e.align4.end(), i) != e.align4.end();
        p[i] = (char *)p[i] + (four ? 2 : 8);
        expect(n + " misaligned arg " + std::to_string(i), e.call(p, s0), ATTN_ERR_MISALIGNED);
    }
    // every output on top of every other argument, and one that starts 16 bytes before another ends
    for (int o : e.outputs) {
        for (int i = 0; i < e.nptr; ++i) {
            if (i == o) continue;
            fill(p, e.nptr);
            p[o] = p[i];
            expect(n + " arg " + std::to_string(o) + " over arg " + std::to_string(i), e.call(p, s0),
                   ATTN_ERR_ALIAS);
        }
        fill(p, e.nptr);
        p[o] = (char *)p[(o + 1) % e.nptr] - 16;
        expect(n + " arg " + std::to_string(o) + " runs into the next", e.call(p, s0), ATTN_ERR_ALIAS);
    }

    // sizes: negative, and products past the documented limits, one argument at a time and all together
    const int big[] = {INT_MAX, INT_MAX - 1, 1 << 30, INT_MIN, -1};
    for (int v : big) {
        for (int f = 0; f < 5; ++f) {
            Sizes s = s0;
            int *field[] = {&s.B, &s.H, &s.Hk, &s.Nq, &s.Nk};
            if (e.one_length && (f == 2 || f == 4)) continue;
            *field[f] = v;
            if (e.one_length) {
                s.Hk = s.H;
                s.Nk = s.Nq;
            }
            // a huge but valid B or H with small N could pass validation: pair every size with a huge N
            if (v > 0 && f < 3) s.Nq = s.Nk = INT_MAX;
            if (v > 0 && f == 2) s.H = s.Hk;
            fill(p, e.nptr);
            expect(n + " size field " + std::to_string(f) + " = " + std::to_string(v), e.call(p, s),
                   ATTN_ERR_BAD_SHAPE);
        }
    }
    {
        Sizes s = s0;
        s.B = s.H = s.Hk = s.Nq = s.Nk = INT_MAX;
        s.d = (n == "attn_fwd_fp8") ? 128 : 256;
        fill(p, e.nptr);
        expect(n + " every size INT_MAX", e.call(p, s), ATTN_ERR_BAD_SHAPE);
    }
    if (!e.one_length) {
        Sizes s = s0;
        s.H = 3;
        s.Hk = 2;
        fill(p, e.nptr);
        expect(n + " H not a multiple of Hk", e.call(p, s), ATTN_ERR_BAD_SHAPE);
        s.H = 2;
        s.Hk = 0;
        expect(n + " Hk = 0 under H = 2", e.call(p, s), ATTN_ERR_BAD_SHAPE);
    }
    // head dimensions outside the supported set
    for (int d : {0, -64, 32, 80, 96, 127, 129, 320, INT_MAX, INT_MIN}) {
        Sizes s = s0;
        s.d = d;
        fill(p, e.nptr);
        expect(n + " d = " + std::to_string(d), e.call(p, s), ATTN_ERR_UNSUPPORTED_D);
    }
    if (n == "attn_fwd_fp8")
        for (int d : {192, 256}) {
            Sizes s = s0;
            s.d = d;
            fill(p, e.nptr);
            expect(n + " d = " + std::to_string(d), e.call(p, s), ATTN_ERR_UNSUPPORTED_D);
        }
    if (e.has_scale)
        for (float sc : {0.0f, -0.125f, std::numeric_limits<float>::infinity(),
                         std::numeric_limits<float>::quiet_NaN(), -std::numeric_limits<float>::infinity()}) {
            Sizes s = s0;
            s.scale = sc;
            fill(p, e.nptr);
            expect(n + " scale " + std::to_string(sc), e.call(p, s), ATTN_ERR_BAD_SCALE);
        }
    if (e.has_causal)
        for (int c : {2, -1, INT_MAX}) {
            Sizes s = s0;
            s.causal = c;
            fill(p, e.nptr);
            expect(n + " causal " + std::to_string(c), e.call(p, s), ATTN_ERR_BAD_ARG);
        }
    if (e.has_splits)
        for (int ns : {0, -1, 257, INT_MAX, INT_MIN}) {
            Sizes s = s0;
            s.ns = ns;
            s.wsb = 1LL << 40;
            fill(p, e.nptr);
            expect(n + " num_splits " + std::to_string(ns), e.call(p, s), ATTN_ERR_BAD_ARG);
        }
    // an empty batch is valid and touches nothing, with every pointer NULL
    {
        Sizes s = s0;
        s.B = 0;
        for (int i = 0; i < e.nptr; ++i) p[i] = nullptr;
        expect(n + " empty batch", e.call(p, s), ATTN_OK);
    }
}

void check_splitkv_sizes()
{
    void *p[6];
    fill(p, 6);
    Sizes s;
    s.Hk = 2;
    const long long need = attn_fwd_splitkv_workspace_size(s.B, s.H, s.Nq, s.d, s.ns);
    expect("workspace size formula", need == (long long)s.ns * s.B * s.H * s.Nq * (s.d + 1) * 4 ? 0 : 1, 0);
    s.wsb = need - 1;
    expect("workspace one byte short", attn_fwd_splitkv(p[0], p[1], p[2], p[3], (float *)p[4], s.B, s.H, s.Hk, s.Nq,
                                                         s.Nk, s.d, s.causal, s.scale, s.ns, p[5], s.wsb, nullptr),
           ATTN_ERR_WORKSPACE);
    // the size helpers at extreme arguments: no overflow, -1 where the size is not representable
    const int vals[] = {INT_MIN, -1, 0, 1, 64, 1 << 20, INT_MAX};
    for (int b : vals)
        for (int h : vals)
            for (int nq : vals)
                for (int d : {64, 128, 192, 256, 80}) {
                    const long long w = attn_fwd_splitkv_workspace_size(b, h, nq, d, 256);
                    const int ds = attn_fwd_splitkv_default_splits(b, h, nq, INT_MAX, d);
                    ++g_calls;
                    if (w < -1 || ds < 1 || ds > 256) {
                        ++g_fail;
                        std::fprintf(stderr, "MISMATCH size helpers at %d %d %d %d: %lld %d\n", b, h, nq, d, w, ds);
                    }
                    for (int hk : vals) {
                        const int dq = attn_fwd_splitkv_default_splits_qk(b, h, hk, nq, INT_MAX, d);
                        ++g_calls;
                        if (dq < 1 || dq > 256) {
                            ++g_fail;
                            std::fprintf(stderr, "MISMATCH default splits at %d %d %d %d %d: %d\n", b, h, hk, nq, d, dq);
                        }
                    }
                }
    // the no-allocation variant: the first size past its static buffer
    Sizes t;
    t.B = 1;
    t.H = t.Hk = 1;
    t.Nq = 8129;
    t.d = 128;
    t.ns = 4;
    expect("noalloc past the buffer", attn_fwd_splitkv_noalloc(nullptr, p[1], p[2], p[3], (float *)p[4], t.B, t.H, t.Hk,
                                                                 t.Nq, t.Nk, t.d, 0, t.scale, t.ns, nullptr),
           ATTN_ERR_SCRATCH);
}

void check_status_strings()
{
    for (int c = -1000; c <= 1000; ++c) {
        const char *str = attn_status_string(c);
        ++g_calls;
        if (!str || !std::strlen(str)) ++g_fail;
    }
    for (int c : {INT_MIN, INT_MAX}) {
        ++g_calls;
        if (!attn_status_string(c)) ++g_fail;
    }
    ++g_calls;
    if (attn_last_hip_error() != 0) ++g_fail;
}

}  // namespace

int main()
{
    for (const Entry &e : entries()) check_entry(e);
    check_splitkv_sizes();
    check_status_strings();
    std::printf("abi checks: %d calls, %d mismatches\n", g_calls, g_fail);
    return g_fail ? 1 : 0;
}
