// Decode step for bf16 io (gfx950): one one-token update interval per
// (sequence, KV head) chain, one workgroup of 8 waves per chain (waves 0-3 read,
// waves 4-7 manage, side by side), state read and written in place.
//
//   read   -- the chain's G query heads (MFMA columns) attend with exact
//             softmax to the window [t-w+1, t] and the cache, streamed in
//             groups of 32 keys dealt to the 4 read waves, with an online
//             softmax per wave, merged at the end; the linear part is H^T phi(q) / s . phi(q)
//             plus the key at t-w that leaves the window at this step (the new
//             key itself when w = 0); one shared denominator (LoLA summary,
//             "Inferentiestrategie", step 4).
//   manage -- the SRE equation ("Het Self-Recall Error (SRE) Mechanisme") for
//             every cached key and the leaving key against the step-start
//             state: the cached keys' features are recomputed from their
//             stored z = W k (written when each key entered the cache: half the
//             bytes of stored hi/lo feature rows), phi(k) = [softmax(z); softmax(-z)];
//             the leaving key's z is computed by MFMA with W in three bf16 parts; n^T = H^T phi^T with H and
//             phi in bf16 hi/lo parts, d = phi . s (s in three bf16 parts); then the pair with the
//             lowest SRE (newest on a tie) is folded into H, s by one outer
//             product when the candidates exceed the capacity, and the leaving
//             key takes its cache slot with its z.
#pragma once

#include <type_traits>

#include "lola_output.h"

namespace lola {

constexpr int kDecBlock = 128;  // V^T staging columns: 32 keys per read wave

struct DecSmem {
    size_t HhT, HlT, Wl, sP, sParts, cposL, esc, phiE, phiF, xrow, stVT, nE, zE, misc, total;
};

// The two arrays sized by the cache capacity come last: every other offset is a
// compile-time constant.
template <int D, int F>
__host__ __device__ constexpr DecSmem dec_smem(int C)
{
    DecSmem m{};
    const int Cp = C > 0 ? C : 1;
    size_t off = 0;
    m.HhT = off;   off += align_up(sizeof(uint16_t) * (size_t)D * (F + 8), 16);
    m.HlT = off;   off += align_up(sizeof(uint16_t) * (size_t)D * (F + 8), 16);
    m.Wl = off;    off += align_up(sizeof(uint16_t) * 3 * (size_t)(F / 2) * (D + 8), 16);  // W parts, padded rows
    m.sP = off;    off += align_up(sizeof(float) * F, 16);
    m.sParts = off; off += align_up(sizeof(uint16_t) * 3 * F, 16);  // s in three bf16 parts, operand order
    m.phiE = off;  off += align_up(sizeof(float) * F, 16);
    m.phiF = off;  off += align_up(sizeof(float) * F, 16);
    m.xrow = off;  off += align_up(sizeof(float) * D, 16);
    m.stVT = off;  off += align_up(sizeof(uint16_t) * (size_t)D * (kDecBlock + 8), 16);
    m.nE = off;    off += align_up(sizeof(float) * (D + 4), 16);   // incremental decode: n, d of the leaving key
    m.zE = off;    off += align_up(sizeof(float) * (F / 2), 16);  // z = W k of the leaving key
    m.misc = off;  off += align_up(sizeof(int) * 16, 16);
    m.cposL = off; off += align_up(sizeof(int) * (size_t)Cp, 16);
    m.esc = off;   off += align_up(sizeof(float) * (size_t)(Cp + 1), 16);
    m.total = align_up(off, 16);
    return m;
}

// z^T = W K^T of P tiles of 16 keys (key r16 of tile p in column r16 of kb[p]) by
// MFMA with W in three bf16 parts (exact products against bf16 keys, fp32 sums; the
// W operands are read once for all P tiles): lane (r16, qg) gets features
// ft * 16 + 4 qg + i of key r16 in zt[p][ft][i].
template <int D, int F, int P>
__device__ __forceinline__ void z_tiles(const uint16_t* Wl, const bf16x8 (*kb)[D / 32], int r16, int qg,
                                        floatx4 (*zt)[F / 32])
{
    constexpr int Fh = F / 2, DS = D / 32, WS = D + 8;  // Wl: [3][Fh][WS] in LDS
#pragma unroll
    for (int ft = 0; ft < Fh / 16; ++ft) {
#pragma unroll
        for (int p = 0; p < P; ++p) zt[p][ft] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DS; ++ks) {
            const int o = (ft * 16 + r16) * WS + ks * 32 + qg * 8;
            const bf16x8 w0 = *(const bf16x8*)(Wl + o), w1 = *(const bf16x8*)(Wl + Fh * WS + o),
                         w2 = *(const bf16x8*)(Wl + 2 * Fh * WS + o);
#pragma unroll
            for (int p = 0; p < P; ++p) {
                zt[p][ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, kb[p][ks], zt[p][ft], 0, 0, 0);
                zt[p][ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, kb[p][ks], zt[p][ft], 0, 0, 0);
                zt[p][ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2, kb[p][ks], zt[p][ft], 0, 0, 0);
            }
        }
    }
}

// phi = [softmax(z); softmax(-z)] from z in the layout z_tiles leaves it (the four
// lanes of a key combine by lane swaps).  x[p][h] is the feature of operand slot h:
// slot h = 8 mf + j holds feature 16 (2 mf + j / 4) + 4 qg + j % 4 (positive half for
// mf < F / 64).  The same arithmetic, in the same order, as the prefill prologue, so
// that phi recomputed from a stored z equals the prologue's phi bit for bit.
template <int F, int P>
__device__ __forceinline__ void phi_from_z(const floatx4 (*zt)[F / 32], float (*x)[F / 4])
{
    constexpr int Fh = F / 2;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float zmax = -INFINITY, zmin = INFINITY;
#pragma unroll
        for (int ft = 0; ft < Fh / 16; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) { zmax = fmaxf(zmax, zt[p][ft][i]); zmin = fminf(zmin, zt[p][ft][i]); }
        zmax = quad_max(zmax);
        zmin = quad_min(zmin);
        float sp = 0.f, sn = 0.f;
#pragma unroll
        for (int ft = 0; ft < Fh / 16; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e1 = exp_acc(zt[p][ft][i] - zmax), e2 = exp_acc(zmin - zt[p][ft][i]);
                x[p][(ft >> 1) * 8 + (ft & 1) * 4 + i] = e1;
                x[p][Fh / 4 + (ft >> 1) * 8 + (ft & 1) * 4 + i] = e2;
                sp += e1;
                sn += e2;
            }
        sp = quad_sum(sp);
        sn = quad_sum(sn);
        const float isp = 1.f / sp, isn = 1.f / sn;
#pragma unroll
        for (int h = 0; h < F / 4; ++h) x[p][h] *= h < Fh / 4 ? isp : isn;
    }
}

// stored z of key `row` (natural feature order, Fh floats) in the z_tiles layout
template <int F>
__device__ __forceinline__ void load_z(const float* row, int qg, floatx4* zt)
{
#pragma unroll
    for (int ft = 0; ft < F / 32; ++ft) {
        const float4 z4 = *(const float4*)(row + ft * 16 + qg * 4);
        zt[ft] = floatx4{z4.x, z4.y, z4.z, z4.w};
    }
}

// bf16 hi / lo operand parts of the features in slot order
template <int F>
__device__ __forceinline__ void hilo_split(const float* x, bf16x8* bh, bf16x8* bl)
{
#pragma unroll
    for (int mf = 0; mf < F / 32; ++mf) {
        u16x8 uh, ul;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float xv = x[mf * 8 + j];
            const uint16_t h = bf16_bits(xv);
            uh[j] = h;
            ul[j] = bf16_bits(xv - bf16_val(h));
        }
        bh[mf] = __builtin_bit_cast(bf16x8, uh);
        bl[mf] = __builtin_bit_cast(bf16x8, ul);
    }
}

// feature index of operand slot h (see phi_tile) for lane group qg
__device__ __forceinline__ int slot_feature(int h, int qg) { return (2 * (h >> 3) + ((h & 7) >> 2)) * 16 + qg * 4 + (h & 3); }

// Waves 0..3 run the read, waves 4..7 the management: both read only the step-start
// state, so the softmax stream over window and cache and the SRE pass over the cache
// run side by side on the same CU instead of one after the other.
constexpr int kDecThreads = 512;

template <int D, int F, bool INC>
__global__ __launch_bounds__(kDecThreads, 1) void decode_kernel_bf16(Args a)
{
    constexpr int NT = kDecThreads, NA = 4, NB = NT / 64 - NA;  // read waves, management waves
    constexpr int LASTW = NT / 64 - 1;                           // the leaving key's wave
    constexpr int Fh = F / 2, FM = F / 32, DS = D / 32, DT = D / 16;
    constexpr int KW = 32;  // keys per step of a read wave
    constexpr int HP = F + 8, VP = kDecBlock + 8;
    static_assert(NA * KW == kDecBlock, "the V^T staging area has one 32-key column block per read wave");
    static_assert(D * F / 4 % NT == 0, "H loads cover the state exactly");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    if (!state_ok(a)) return;  // header mismatch or faulted state: nothing is read or written
    const Dims& d = a.d;
    const int G = d.G, w = d.w, C = d.C;
    const DecSmem sm = dec_smem<D, F>(C);  // only the last two offsets depend on C
    uint16_t* HhT = (uint16_t*)(smem + sm.HhT);
    uint16_t* HlT = (uint16_t*)(smem + sm.HlT);
    float* sP = (float*)(smem + sm.sP);
    uint16_t* sParts = (uint16_t*)(smem + sm.sParts);
    int* cposL = (int*)(smem + sm.cposL);
    float* esc = (float*)(smem + sm.esc);
    float* phiE = (float*)(smem + sm.phiE);
    float* phiF = (float*)(smem + sm.phiF);
    float* xrow = (float*)(smem + sm.xrow);
    uint16_t* Wl = (uint16_t*)(smem + sm.Wl);
    uint16_t* stVT = (uint16_t*)(smem + sm.stVT);
    int* misc = (int*)(smem + sm.misc);
    float* mrg = (float*)(smem + sm.stVT);  // merge area, reused after the key loop
    float* nEL = (float*)(smem + sm.nE);    // incremental decode: n of the leaving key, then d at [D]
    float* zE = (float*)(smem + sm.zE);

    const int chain = blockIdx.x, b = chain / d.Hkv, g = chain % d.Hkv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, qg = lane >> 4;
    const bool rd = wave < NA;  // a read wave
    Chain ch = chain_of(a, chain);
    const int64_t t = ch.tok();
    const int cnt = min(max(ch.cnt(), 0), C);
    // incremental decode: the stored n = H^T phi(k), d = s . phi(k) of the cached pairs
    // match the state (a prefill call marks them stale)
    const bool incValid = INC && ch.incv() == 1;
    const bf16* knew = (const bf16*)a.k + ((size_t)b * d.Hkv + g) * D;
    const bf16* vnew = (const bf16*)a.v + ((size_t)b * d.Hkv + g) * D;
    const bool hasE = (w == 0) || (t - w >= 0);
    const int64_t pE = t - w;
    const int rs = w > 0 ? (int)(t % w) : 0;
    const bf16* kE = w == 0 ? knew : ch.ring_k<bf16>() + (size_t)rs * D;
    const bf16* vE = w == 0 ? vnew : ch.ring_v<bf16>() + (size_t)rs * D;
    const uint16_t* Wb = (const uint16_t*)(a.state + a.sl.Wb) + (size_t)(3 * g) * Fh * D;
    const int nU = cnt + (hasE ? 1 : 0);
    const bool foldStep = hasE && nU > C;

    // ---- keys of the read: window [ws0, t] then cache slots, in groups of 32 ----
    const int64_t ws0 = t - w + 1 > 0 ? t - w + 1 : 0;
    const int nWin = w > 0 ? (int)(t - ws0 + 1) : 0;
    const int nK = nWin + cnt;
    // row of key kidx (0 <= kidx < nK): window position ws0 + kidx (ring slot
    // (ws0 + kidx) mod w, the newest being this step's token), then cache slot
    // kidx - nWin; chosen by selects so that a group's loads issue together
    const int rs0 = w > 0 ? (int)(ws0 % w) : 0;
    auto key_row = [&](int kidx, bool v) -> const bf16* {
        int slot = rs0 + kidx;
        slot = slot >= w ? slot - w : slot;
        const bf16* pw = (v ? ch.ring_v<bf16>() : ch.ring_k<bf16>()) + (size_t)slot * D;
        const bf16* pc = (v ? ch.cache_v<bf16>() : ch.cache_k<bf16>()) + (ptrdiff_t)(kidx - nWin) * D;
        const bf16* pn = v ? vnew : knew;
        return kidx < nWin ? (kidx == nWin - 1 ? pn : pw) : pc;
    };
    const int ng = (nK + KW - 1) / KW;
    // groups are dealt to the read waves in turn, wave 0 (which first computes phi(q)
    // and the linear read) taking the last group of each round
    const int g0 = (wave + NA - 1) % NA;
    // A read wave loads its group's key fragments (keys 32 g + tt * 16 + r16, 16 bytes
    // per lane straight from the key row) and value rows (lane: key pair lane % 16,
    // 8-value units lane / 16 + 4 j); rows past nK load the last key and are zeroed.
    constexpr int VNW = (KW / 2) * (D / 8) / 64;
    static_assert((KW / 2) * (D / 8) % 64 == 0, "value units cover a group exactly");
    uint4 kq[2][DS], vqa[VNW], vqb[VNW];
    auto issue = [&](int gg) {
        const int base = gg * KW;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int kidx = base + tt * 16 + r16;
            const bf16* kr = key_row(kidx < nK ? kidx : nK - 1, false);
#pragma unroll
            for (int ks = 0; ks < DS; ++ks) kq[tt][ks] = *(const uint4*)(kr + ks * 32 + qg * 8);
        }
#pragma unroll
        for (int j = 0; j < VNW; ++j) {
            const int k0 = base + 2 * r16, un = qg + 4 * j;
            vqa[j] = *(const uint4*)(key_row(k0 < nK ? k0 : nK - 1, true) + un * 8);
            vqb[j] = *(const uint4*)(key_row(k0 + 1 < nK ? k0 + 1 : nK - 1, true) + un * 8);
        }
    };

    // ---- SRE pass over the cache (management waves): to choose a victim, or
    //      (incremental decode) to compute the stored n, d of every cached pair afresh ----
    const bool scoreCache = INC ? (!incValid && cnt > 0) : foldStep;
    const bool storedScores = INC && incValid && foldStep;
    const int nT = (cnt + 15) / 16;
    const int bw = wave - NA;
    // the cached keys' features are recomputed from their stored z = W k (Fh floats
    // per key, a quarter of them per lane in the z_tiles layout)
    floatx4 zq[F / 32];
    uint2 vq[DT];
    auto tile_load = [&](int tt) {
        const int slot = tt * 16 + r16 < cnt ? tt * 16 + r16 : cnt - 1;
        load_z<F>(ch.cz() + (size_t)slot * Fh, qg, zq);
        const bf16* vr = ch.cache_v<bf16>() + (size_t)slot * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vq[dt] = *(const uint2*)(vr + dt * 16 + qg * 4);
    };

    // ---- state in: H^T hi/lo in operand order, W parts, s, cache positions ----
    {
        const float* Hst = ch.H();  // [D][F]
        constexpr int HN = D * F / 4 / NT;  // float4 per thread, all loaded before any is used
        constexpr int WTOT = 3 * Fh * D / 8, WN = (WTOT + NT - 1) / NT;  // 16-byte pieces of the W parts
        // W parts to LDS in batches of WB pieces (all loads of a batch issued before any
        // is stored); H (from HBM, the longest wait) is requested first, all of it, and
        // the W batches (L2 hits) are stored to LDS while it is in flight
        constexpr int WB = WN % 3 == 0 ? 3 : (WN % 2 == 0 ? 2 : 1);
        float4 hv4[HN];
#pragma unroll
        for (int k = 0; k < HN; ++k) hv4[k] = *(const float4*)(Hst + (size_t)(tid + k * NT) * 4);
#pragma unroll
        for (int k0 = 0; k0 < WN; k0 += WB) {
            uint4 w4[WB];
#pragma unroll
            for (int k = 0; k < WB; ++k) {
                const int pc = tid + (k0 + k) * NT;
                w4[k] = pc < WTOT ? *(const uint4*)(Wb + (size_t)pc * 8) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int k = 0; k < WB; ++k) {
                const int pc = tid + (k0 + k) * NT;
                const int e = pc * 8, row = e / D, col = e % D;  // row = part * Fh + feature
                if (pc < WTOT) *(uint4*)(Wl + row * (D + 8) + col) = w4[k];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int k = 0; k < HN; ++k) {
            const int i = tid + k * NT, dd = (i * 4) / F, f = (i * 4) % F;
            const float vv[4] = {hv4[k].x, hv4[k].y, hv4[k].z, hv4[k].w};
            uint16_t h[4], l[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h[j] = bf16_bits(vv[j]);
                l[j] = bf16_bits(vv[j] - bf16_val(h[j]));
            }
            const int o = dd * HP + perm_pos(f);  // four consecutive features stay consecutive
            *(uint2*)(HhT + o) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
            *(uint2*)(HlT + o) = make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
        }
        for (int i = tid; i < F; i += NT) {
            const float x = ch.s()[i];
            const int o = perm_pos(i);
            sP[o] = x;
            const uint16_t p1 = bf16_bits(x);
            const float r1 = x - bf16_val(p1);
            const uint16_t p2 = bf16_bits(r1);
            sParts[o] = p1;
            sParts[F + o] = p2;
            sParts[2 * F + o] = bf16_bits(r1 - bf16_val(p2));
        }
        for (int i = tid; i < cnt; i += NT) cposL[i] = ch.cpos()[i];
        if (tid == 0) {
            misc[1] = 0;   // set once the leaving key's features are in LDS
            misc[2] = NB;  // next cache tile to score (tiles 0 .. NB - 1 go to the management waves)
        }
    }
    // query frags (read waves, columns r16 < G); the leaving key's row (last wave,
    // column 0) and its value rows dt * 16 + 4 qg .. + 3 (wave 0 and the last wave)
    bf16x8 qf[DS];
    uint4 kEq[DS];
    uint2 vEq[DT];
    {
        const bool le = hasE && (wave == 0 || wave == LASTW);
#pragma unroll
        for (int ks = 0; ks < DS; ++ks)
            kEq[ks] = (hasE && wave == LASTW && r16 == 0) ? *(const uint4*)(kE + ks * 32 + qg * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vEq[dt] = le ? *(const uint2*)(vE + dt * 16 + qg * 4) : make_uint2(0, 0);
        const bool qv = rd && r16 < G;
        const bf16* qp = (const bf16*)a.q + ((size_t)b * d.Hq + g * G + (qv ? r16 : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < DS; ++ks) {
            const uint4 u4 = qv ? *(const uint4*)(qp + ks * 32 + qg * 8) : make_uint4(0, 0, 0, 0);
            qf[ks] = __builtin_bit_cast(bf16x8, u4);
        }
    }
    __syncthreads();  // W parts and H in LDS
    // the first group of keys (read waves) and the first cache tiles (management waves)
    if (rd) {
        if (g0 < ng) issue(g0);
    } else if (scoreCache && bw < nT) {
        tile_load(bw);
    }
    // Error of P tiles of 16 candidates from their feature operands (bf16 hi, lo
    // parts bh, bl; candidate r16 of tile p) and 1 / d: n^T = H^T phi^T with H and phi
    // in hi/lo parts (hi.hi + lo.hi + hi.lo; the H operands are read once for all P
    // tiles), e = |n / d - v|^2 (values vq[p] at rows dt * 16 + 4 qg .. + 3)
    // (nout[p], if given, receives candidate r16's n at its rows dt * 16 + 4 qg .. + 3)
    auto sre_core = [&](auto pTag, const bf16x8 (*bh)[FM], const bf16x8 (*bl)[FM], const float* inv,
                        const uint2 (*vqq)[DT], float* e, float* const* nout = nullptr) {
        constexpr int P = decltype(pTag)::value;
        float es[P];
#pragma unroll
        for (int p = 0; p < P; ++p) es[p] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            floatx4 acc[P], acc2[P];
#pragma unroll
            for (int p = 0; p < P; ++p) acc[p] = acc2[p] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mf = 0; mf < FM; ++mf) {
                const int o = (dt * 16 + r16) * HP + mf * 32 + qg * 8;
                const bf16x8 ah = *(const bf16x8*)(HhT + o);
                const bf16x8 al = *(const bf16x8*)(HlT + o);
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh[p][mf], acc[p], 0, 0, 0);
                    acc2[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh[p][mf], acc2[p], 0, 0, 0);
                    acc2[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl[p][mf], acc2[p], 0, 0, 0);
                }
            }
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const float vv[4] = {__uint_as_float(vqq[p][dt].x << 16), __uint_as_float(vqq[p][dt].x & 0xffff0000u),
                                     __uint_as_float(vqq[p][dt].y << 16), __uint_as_float(vqq[p][dt].y & 0xffff0000u)};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float df = (acc[p][i] + acc2[p][i]) * inv[p] - vv[i];
                    es[p] += df * df;
                }
                if (nout && nout[p])
                    *(float4*)(nout[p] + dt * 16 + qg * 4) = make_float4(acc[p][0] + acc2[p][0], acc[p][1] + acc2[p][1],
                                                                         acc[p][2] + acc2[p][2], acc[p][3] + acc2[p][3]);
            }
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            es[p] = quad_sum(es[p]);
            e[p] = es[p];
        }
    };
    // d = s . (phi hi + phi lo), the feature values the MFMAs see, by MFMA as in the
    // prefill scan: A rows 4q, 4q + 1, 4q + 2 hold the three bf16 parts of s (row
    // 4q + 3 zero), so every lane group receives d of its column (candidate r16) in
    // its own result rows; the products are exact and the sums fp32
    auto dot_s = [&](const bf16x8* bh, const bf16x8* bl) -> float {
        const int row = (r16 & 3) < 3 ? (r16 & 3) : 2;
        const uint32_t keepm = (r16 & 3) < 3 ? 0xffffffffu : 0u;
        floatx4 dac = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mf = 0; mf < FM; ++mf) {
            uint4 x = *(const uint4*)(sParts + row * F + mf * 32 + qg * 8);
            x.x &= keepm;
            x.y &= keepm;
            x.z &= keepm;
            x.w &= keepm;
            const bf16x8 as = __builtin_bit_cast(bf16x8, x);
            dac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as, bh[mf], dac, 0, 0, 0);
            dac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as, bl[mf], dac, 0, 0, 0);
        }
        return (dac[0] + dac[1]) + dac[2];
    };

    floatx4 O[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mrun = 0.f, Zp = 0.f;
    const float tau = d.tau;
    if (rd) {
        if (wave == 0) {
            // phi(q) for the query columns: z^T = W Q^T with W hi + lo, then the linear
            // read O_lin^T = H^T phi(q)^T and s . phi(q)
            float xq[F / 4];  // phi(q) of column r16, operand-slot order
            float zq = 0.f;
            floatx4 zt[Fh / 16];
#pragma unroll
            for (int ft = 0; ft < Fh / 16; ++ft) {
                zt[ft] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < DS; ++ks) {
                    const int o = (ft * 16 + r16) * (D + 8) + ks * 32 + qg * 8;
                    zt[ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(Wl + o), qf[ks], zt[ft], 0, 0, 0);
                    zt[ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(Wl + Fh * (D + 8) + o), qf[ks], zt[ft], 0, 0, 0);
                }
            }
            float zmax = -INFINITY, zmin = INFINITY;
#pragma unroll
            for (int ft = 0; ft < Fh / 16; ++ft)
#pragma unroll
                for (int i = 0; i < 4; ++i) { zmax = fmaxf(zmax, zt[ft][i]); zmin = fminf(zmin, zt[ft][i]); }
            zmax = quad_max(zmax);
            zmin = quad_min(zmin);
            float sp = 0.f, sn = 0.f;
#pragma unroll
            for (int ft = 0; ft < Fh / 16; ++ft)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e1 = __expf(zt[ft][i] - zmax), e2 = __expf(zmin - zt[ft][i]);
                    xq[(ft >> 1) * 8 + (ft & 1) * 4 + i] = e1;
                    xq[Fh / 4 + (ft >> 1) * 8 + (ft & 1) * 4 + i] = e2;
                    sp += e1;
                    sn += e2;
                }
            sp = quad_sum(sp);
            sn = quad_sum(sn);
            const float isp = 1.f / sp, isn = 1.f / sn;
            bf16x8 pf[FM];
#pragma unroll
            for (int mf = 0; mf < FM; ++mf) {
                u16x8 u;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int hidx = mf * 8 + j;
                    xq[hidx] *= hidx < Fh / 4 ? isp : isn;
                    u[j] = bf16_bits(xq[hidx]);
                    zq += xq[hidx] * sP[mf * 32 + qg * 8 + j];  // operand position of this feature
                }
                pf[mf] = __builtin_bit_cast(bf16x8, u);
            }
            zq = quad_sum(zq);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int mf = 0; mf < FM; ++mf)
                    O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(HhT + (dt * 16 + r16) * HP + mf * 32 + qg * 8),
                                                                    pf[mf], O[dt], 0, 0, 0);
            // the leaving key's linear weight kappa = phi(q) . phi(k_E) per query column;
            // kappa * v_E joins the linear part (weight e^-M, M floored at 0).  Its
            // features come from the last wave through LDS: wait for its flag (a bounded
            // poll; the last wave sets the flag without waiting for anything)
            {
                int it = 0;
                while (__hip_atomic_load(&misc[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0 && it < (1 << 22)) {
                    __builtin_amdgcn_s_sleep(1);
                    ++it;
                }
                if (it >= (1 << 22) && lane == 0)
                    __hip_atomic_store(&((StateHeader*)a.state)->fault, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
            }
            float kap = 0.f;
#pragma unroll
            for (int mf = 0; mf < FM; ++mf)
#pragma unroll
                for (int j = 0; j < 8; ++j) kap += xq[mf * 8 + j] * phiE[(2 * mf + (j >> 2)) * 16 + qg * 4 + (j & 3)];
            kap = quad_sum(kap);
            if (!hasE) kap = 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const float vv[4] = {__uint_as_float(vEq[dt].x << 16), __uint_as_float(vEq[dt].x & 0xffff0000u),
                                     __uint_as_float(vEq[dt].y << 16), __uint_as_float(vEq[dt].y & 0xffff0000u)};
#pragma unroll
                for (int i = 0; i < 4; ++i) O[dt][i] += kap * vv[i];
            }
            Zp = qg == 0 ? zq + kap : 0.f;
        }

        // ---- this wave's groups of 32 keys: the next group loads while the current
        //      one is scored; V^T is staged in the wave's own 32 columns of the staging
        //      area, so no other wave is waited for ----
        for (int gg = g0; gg < ng; gg += NA) {
            const int base = gg * KW;
            uint4 kcur[2][DS], va[VNW], vb[VNW];  // this group's rows (kq, vqa, vqb are refilled below)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int ks = 0; ks < DS; ++ks) kcur[tt][ks] = base + tt * 16 + r16 < nK ? kq[tt][ks] : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < VNW; ++j) {
                va[j] = base + 2 * r16 < nK ? vqa[j] : make_uint4(0, 0, 0, 0);
                vb[j] = base + 2 * r16 + 1 < nK ? vqb[j] : make_uint4(0, 0, 0, 0);
            }
            if (gg + NA < ng) issue(gg + NA);
            // V^T of the group: LDS runs one wave's instructions in order, so these stores
            // land after the previous group's reads of the same columns and before this
            // group's reads (the asm keeps the compiler from moving LDS accesses across)
            asm volatile("" ::: "memory");
            const int kc = wave * KW + key_perm(2 * r16);
#pragma unroll
            for (int j = 0; j < VNW; ++j) {
                const int un = qg + 4 * j;
                const uint32_t w0[4] = {va[j].x, va[j].y, va[j].z, va[j].w}, w1[4] = {vb[j].x, vb[j].y, vb[j].z, vb[j].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t lo = (w0[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    const uint32_t hi = (w1[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    *(uint32_t*)(stVT + (un * 8 + e) * VP + kc) = lo | (hi << 16);
                }
            }
            lds_wait();
            asm volatile("" ::: "memory");
            floatx4 sT[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                sT[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < DS; ++ks)
                    sT[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kcur[tt][ks]), qf[ks], sT[tt], 0, 0, 0);
            }
            // online softmax for the query column r16 over the lane's 8 keys
            float lg[8];
            bool ok[8];
            float bmax = -INFINITY;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int tt = j >> 2, i = j & 3;
                const int kidx = base + tt * 16 + qg * 4 + i;
                ok[j] = kidx < nK && r16 < G;
                lg[j] = tau * sT[tt][i];
                if (ok[j]) bmax = fmaxf(bmax, lg[j]);
            }
            bmax = quad_max(bmax);
            const float mnew = fmaxf(mrun, bmax);
            const float resc = __expf(mrun - mnew);
            mrun = mnew;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) O[dt] *= resc;
            Zp *= resc;
            u16x8 u;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float pv = ok[j] ? __expf(lg[j] - mnew) : 0.f;
                Zp += pv;
                u[j] = bf16_bits(pv);
            }
            const bf16x8 pb = __builtin_bit_cast(bf16x8, u);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(stVT + (dt * 16 + r16) * VP + wave * KW + qg * 8),
                                                                pb, O[dt], 0, 0, 0);
        }
    } else {
        // ---- management waves ----
        if (wave == LASTW) {
            // phi of the leaving key (column 0 of a tile), handed to wave 0 through LDS,
            // then, when a pair must be folded (or, incremental decode, the key may enter
            // the cache with its n, d), its SRE against the step-start state
            bf16x8 kb[1][DS];
#pragma unroll
            for (int ks = 0; ks < DS; ++ks) kb[0][ks] = __builtin_bit_cast(bf16x8, kEq[ks]);
            floatx4 zt[1][F / 32];
            z_tiles<D, F, 1>(Wl, kb, r16, qg, zt);
            float x[1][F / 4];
            phi_from_z<F, 1>(zt, x);
            if (r16 == 0) {
#pragma unroll
                for (int h = 0; h < F / 4; ++h) phiE[slot_feature(h, qg)] = x[0][h];
#pragma unroll
                for (int ft = 0; ft < F / 32; ++ft)
                    *(float4*)(zE + ft * 16 + qg * 4) = make_float4(zt[0][ft][0], zt[0][ft][1], zt[0][ft][2], zt[0][ft][3]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            if (lane == 0) __hip_atomic_store(&misc[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (hasE && (foldStep || INC)) {
                bf16x8 bh[1][FM], bl[1][FM];
                hilo_split<F>(x[0], bh[0], bl[0]);
                const float dd = dot_s(bh[0], bl[0]);
                const float inv[1] = {dd > 0.f ? 1.f / dd : 0.f};
                if (INC && lane == 0) nEL[D] = dd;
                uint2 vqq[1][DT];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) vqq[0][dt] = vEq[dt];
                float* nout[1] = {(INC && r16 == 0) ? nEL : nullptr};
                float e[1];
                sre_core(std::integral_constant<int, 1>{}, bh, bl, inv, vqq, e, nout);
                if (lane == 0) esc[cnt] = e[0];
            }
        }
        if constexpr (INC) {
            if (storedScores) {
                // e = |n / d - v|^2 from the stored n, d: 16 lanes per cached pair, D / 16
                // values each (one 16-lane group reads a contiguous row)
                constexpr int DPL = D / 16;
                const int sub = lane & 15;
                for (int u = ((tid - NA * 64) >> 4); u < cnt; u += NB * 4) {
                    const float dd = ch.cd()[u];
                    const float inv = dd > 0.f ? 1.f / dd : 0.f;
                    const float* nr = ch.cn() + (size_t)u * D + sub * DPL;
                    const bf16* vr = ch.cache_v<bf16>() + (size_t)u * D + sub * DPL;
                    float e = 0.f;
#pragma unroll
                    for (int j = 0; j < DPL; j += 4) {
                        float nv[4], vv[4];
                        load4(nr + j, nv);
                        load4(vr + j, vv);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float df = nv[i] * inv - vv[i];
                            e += df * df;
                        }
                    }
#pragma unroll
                    for (int o = 1; o < 16; o <<= 1) e += __shfl_xor(e, o, 64);
                    if (sub == 0) esc[u] = e;
                }
            }
        }
    }
    // ---- the cache in tiles of 16 slots: each management wave starts with its own
    //      tile, then every wave takes the next unscored tile from an LDS counter as it
    //      frees up (the read waves once their key groups are done); a tile's z and
    //      value rows load while the previous tile is scored ----
    if (scoreCache) {
        auto grab = [&]() -> int {
            int v = 0;
            if (lane == 0) v = __hip_atomic_fetch_add(&misc[2], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return __builtin_amdgcn_readfirstlane(v);
        };
        int tcur = rd ? grab() : bw;
        if (rd && tcur < nT) tile_load(tcur);
        while (tcur < nT) {
            bf16x8 bh[1][FM], bl[1][FM];
            uint2 vv[1][DT];
            // (slots past the count are scored as stored -- zero or an earlier
            // pair's finite row -- and their errors are not kept)
            const bool cv = tcur * 16 + r16 < cnt;
            floatx4 zc[1][F / 32];
#pragma unroll
            for (int ft = 0; ft < F / 32; ++ft) zc[0][ft] = zq[ft];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) vv[0][dt] = vq[dt];
            const int tnext = grab();
            if (tnext < nT) tile_load(tnext);
            {
                float x[1][F / 4];
                phi_from_z<F, 1>(zc, x);
                hilo_split<F>(x[0], bh[0], bl[0]);
            }
            const float dd = dot_s(bh[0], bl[0]);
            const float inv[1] = {dd > 0.f ? 1.f / dd : 0.f};
            float* nout[1] = {nullptr};
            if (INC && cv) {  // the stored n, d of this cached pair, computed afresh
                const int slot = tcur * 16 + r16;
                nout[0] = ch.cn() + (size_t)slot * D;
                if (qg == 0) ch.cd()[slot] = dd;
            }
            float e[1];
            sre_core(std::integral_constant<int, 1>{}, bh, bl, inv, vv, e, nout);
            if (qg == 0 && cv) esc[tcur * 16 + r16] = e[0];
            tcur = tnext;
        }
    }
    // the read's parts are final and the staging area is free; all SRE in LDS (the
    // incremental decode's fresh n, d stores are also visible to the whole workgroup)
    if constexpr (INC) __syncthreads();
    else lds_sync();

    // ---- merge the read waves' softmax parts; choose the victim and fetch its row ----
    constexpr int HN = D * F / 4 / NT;  // float4 of H per thread for the fold
    float4 h4[HN];
    float* Hd = ch.H();
    if (foldStep) {
        // H (fp32) for the fold is requested before the victim is known
#pragma unroll
        for (int k = 0; k < HN; ++k) h4[k] = *(const float4*)(Hd + (size_t)(tid + k * NT) * 4);
    }
    float* mM = mrg;                 // [NA][16]
    float* mZ = mrg + NA * 16;       // [NA][16]
    float* mO = mrg + 2 * NA * 16;   // [NA][D][16]
    if (rd) {
        float Z = Zp;
        Z = quad_sum(Z);
        if (qg == 0) { mM[wave * 16 + r16] = mrun; mZ[wave * 16 + r16] = Z; }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mO[(wave * D + dt * 16 + qg * 4 + i) * 16 + r16] = O[dt][i];
    } else if (foldStep && wave == NA) {
        // lowest SRE, newest position on a tie: minimise (bits(e), ~pos)
        unsigned long long best = ~0ull;
        for (int u = lane; u < nU; u += 64) {
            const uint32_t pos = u < cnt ? (uint32_t)cposL[u] : (uint32_t)pE;
            const unsigned long long key = ((unsigned long long)__float_as_uint(esc[u]) << 32) | (0xffffffffu - pos);
            best = key < best ? key : best;
        }
        for (int o = 32; o > 0; o >>= 1) {
            const unsigned long long other = __shfl_xor(best, o, 64);
            best = other < best ? other : best;
        }
        const uint32_t pos = 0xffffffffu - (uint32_t)(best & 0xffffffffu);
        int vi = cnt;
        for (int u = lane; u < cnt; u += 64)
            if ((uint32_t)cposL[u] == pos) vi = u;
        for (int o = 32; o > 0; o >>= 1) vi = min(vi, __shfl_xor(vi, o, 64));
        if (lane == 0) misc[0] = vi;
        // the folded pair: its features (hi + lo) from its stored z, or the leaving
        // key's features, and its value
        if (vi < cnt) {
            // recomputed from its stored z as the SRE pass computed them (every column
            // of the tile holds the victim; column 0 writes), hi + lo as in the SRE
            floatx4 zt[1][F / 32];
            load_z<F>(ch.cz() + (size_t)vi * Fh, qg, zt[0]);
            float x[1][F / 4];
            phi_from_z<F, 1>(zt, x);
            if (r16 == 0)
#pragma unroll
                for (int h = 0; h < F / 4; ++h) {
                    const uint16_t hb = bf16_bits(x[0][h]);
                    phiF[slot_feature(h, qg)] = bf16_val(hb) + bf16_val(bf16_bits(x[0][h] - bf16_val(hb)));
                }
        } else
            for (int f = lane; f < F; f += 64) phiF[f] = phiE[f];
        const bf16* vr = vi < cnt ? ch.cache_v<bf16>() + (size_t)vi * D : vE;
        for (int j = lane; j < D; j += 64) xrow[j] = to_f32(vr[j]);
    }
    lds_sync();  // merge parts, victim and its rows in LDS (H stays in flight)
    for (int idx = tid; idx < G * D; idx += NT) {
        const int col = idx / D, dd = idx % D;
        float M = 0.f;
#pragma unroll
        for (int ww = 0; ww < NA; ++ww) M = fmaxf(M, mM[ww * 16 + col]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int ww = 0; ww < NA; ++ww) {
            const float sc = __expf(mM[ww * 16 + col] - M);
            num += sc * mO[(ww * D + dd) * 16 + col];
            den += sc * mZ[ww * 16 + col];
        }
        ((bf16*)a.out)[((size_t)b * d.Hq + g * G + col) * D + dd] = from_f32<bf16>(num / den);
    }
    int victim = -1;
    if (foldStep) {
        // H += phi v^T, s += phi
        victim = misc[0];
#pragma unroll
        for (int k = 0; k < HN; ++k) {
            const int i = (tid + k * NT) * 4, dd = i / F, f = i % F;
            const float vv = xrow[dd];
            h4[k].x += vv * phiF[f];
            h4[k].y += vv * phiF[f + 1];
            h4[k].z += vv * phiF[f + 2];
            h4[k].w += vv * phiF[f + 3];
            *(float4*)(Hd + i) = h4[k];
        }
        for (int f = tid; f < F; f += NT) ch.s()[f] += phiF[f];
    }

    if constexpr (INC) {
        // ---- stored n, d after this step: every cached pair that stays gains the folded
        //      pair's share, kappa = phi(k) . phi(k_f) times [v_f; 1] (H += phi_f v_f^T and
        //      s += phi_f leave n = H^T phi(k), d = s . phi(k) exactly that much larger);
        //      a leaving key that enters the cache brings its own n, d (the last wave
        //      computed them against the step-start state) plus its share of the fold ----
        if (foldStep) {
            // tiles of 16 cached pairs dealt to the waves: the pair's features from its
            // stored z as in the SRE pass (hi + lo), kappa = phi . phi_f over the four
            // lanes of its column, then lane group qg adds kappa v_f to n at rows
            // qg * D / 4 .. + D / 4
            constexpr int DQ = D / 4;
            const int nTc = (cnt + 15) / 16;
            for (int tt = wave; tt < nTc; tt += NT / 64) {
                const int u = tt * 16 + r16;
                const bool cv = u < cnt && u != victim;
                floatx4 zt[1][F / 32];
                load_z<F>(ch.cz() + (size_t)(u < cnt ? u : cnt - 1) * Fh, qg, zt[0]);
                float x[1][F / 4];
                phi_from_z<F, 1>(zt, x);
                float kk = 0.f;
#pragma unroll
                for (int h = 0; h < F / 4; ++h) {
                    const uint16_t hb = bf16_bits(x[0][h]);
                    kk += (bf16_val(hb) + bf16_val(bf16_bits(x[0][h] - bf16_val(hb)))) * phiF[slot_feature(h, qg)];
                }
                kk = quad_sum(kk);
                if (cv) {
                    float* nr = ch.cn() + (size_t)u * D + qg * DQ;
#pragma unroll
                    for (int j = 0; j < DQ; j += 4) {
                        float4 n4 = *(const float4*)(nr + j);
                        n4.x += kk * xrow[qg * DQ + j];
                        n4.y += kk * xrow[qg * DQ + j + 1];
                        n4.z += kk * xrow[qg * DQ + j + 2];
                        n4.w += kk * xrow[qg * DQ + j + 3];
                        *(float4*)(nr + j) = n4;
                    }
                    if (qg == 0) ch.cd()[u] += kk;
                }
            }
        }
        const int enter = !hasE ? -1 : (nU <= C ? cnt : (victim < cnt ? victim : -1));
        if (enter >= 0 && wave == 0) {
            float ke = 0.f;
            if (foldStep) {
                for (int f = lane; f < F; f += 64) ke += phiE[f] * phiF[f];
                ke = wave_sum(ke);
            }
            for (int j = lane; j < D; j += 64) ch.cn()[(size_t)enter * D + j] = nEL[j] + (foldStep ? ke * xrow[j] : 0.f);
            if (lane == 0) ch.cd()[enter] = nEL[D] + ke;
        }
    }

    // ---- cache slot, then the ring (the leaving pair lives in slot t % w) ----
    // (the victim's rows were read before the barrier above; each thread reads the
    // leaving pair's elements before it overwrites them, so no barrier waits for the
    // H stores)
    int slot = -1;
    if (hasE) {
        if (nU <= C) slot = cnt;
        else if (victim < cnt) slot = victim;
    }
    if (slot >= 0) {
        for (int j = tid; j < D; j += NT) {
            ch.cache_k<bf16>()[(size_t)slot * D + j] = kE[j];
            ch.cache_v<bf16>()[(size_t)slot * D + j] = vE[j];
        }
        for (int f = tid; f < Fh; f += NT) ch.cz()[(size_t)slot * Fh + f] = zE[f];  // its z = W k
    }
    if (w > 0)
        for (int j = tid; j < D; j += NT) {
            ch.ring_k<bf16>()[(size_t)rs * D + j] = knew[j];
            ch.ring_v<bf16>()[(size_t)rs * D + j] = vnew[j];
        }
    if (tid == 0) {
        if (slot >= 0) ch.cpos()[slot] = (int32_t)pE;
        if (hasE && nU <= C) ch.cnt() = cnt + 1;
        ch.tok() = t + 1;
        if (INC) ch.incv() = 1;
    }
}

}  // namespace lola
