// Output pass for bf16 io (gfx950), LDS-staged.
//
// One workgroup (8 waves) handles 256 query rows of one (interval, chain) --
// all G * L of them at the 4K workload's shapes, so the window, cache and
// snapshot tiles of an interval are staged once; each wave owns 32 rows as two
// 16-column MFMA tiles (the queries are the columns, so softmax statistics live
// in the lanes), and every K, V and phi(K) operand read from LDS feeds both
// tiles.  Per workgroup:
//   - H_c^T (bf16, features in operand order) and W (bf16 hi + lo) staged in LDS
//     once (every load issued before any is waited for);
//   - z^T = W Q^T gives phi(q) (two softmax halves over the features),
//     O^T = H_c^T phi(q)^T and Z = s_c . phi(q) start the accumulators
//     (linear read of the interval-start state, LoLA summary section
//     "Inferentiestrategie", step 4);
//   - keys in blocks of 64 (the window span of the interval, then the cache
//     snapshot): K, V^T and phi(K) are staged in LDS with 16-byte loads, the
//     next block prefetched into registers (the first one before phi(q) is
//     computed), and each block is consumed in two steps of 32 keys so the
//     per-step registers stay those of a 32-key block; S^T = K Q^T, kappa^T = phi(K) phi(q)^T
//     for keys that left the window inside the interval, online softmax
//     against a reference M >= 0 (the linear terms carry e^-M) that moves only
//     when a logit exceeds it by more than 8, so O and Z are rarely rescaled,
//     and O^T += V^T P^T; the blocks past the window span (cache keys only)
//     skip phi(K), kappa and the key classification;
//   - o = O / Z with one shared denominator.
#pragma once

#include "lola_prefill.h"

namespace lola {

constexpr int kOutRows = 256;  // query rows per workgroup
constexpr int kKeyBlock = 64;  // keys staged per block: one load round trip per 64 keys
constexpr int kKeyStep = 32;   // keys per compute step (two row tiles per wave with 64-key steps spill registers)
constexpr float kRescaleGap = 8.f;  // the softmax reference moves when a logit exceeds it by more
constexpr int kOutThreads = 512;  // 8 waves x 32 query rows

struct OutSmem {
    size_t sP, refs, Wl, Hs, Ks, VT, Pk, rowK, rowV, total;
};

// The cache references come last: every other offset is a compile-time constant.
template <int D, int F>
__host__ __device__ constexpr OutSmem out_smem(int C)
{
    OutSmem m{};
    size_t off = 0;
    m.sP = off;   off += align_up(sizeof(float) * F, 16);
    m.Wl = off;   off += align_up(sizeof(uint16_t) * 2 * (size_t)(F / 2) * (D + 8), 16);  // W hi, lo [2][Fh][D+8]
    m.Hs = off;   off += align_up(sizeof(uint16_t) * (size_t)D * (F + 8), 16);            // H_c^T [D][F+8]
    m.Ks = off;   off += sizeof(uint16_t) * (size_t)kKeyBlock * (D + 8);
    m.VT = off;   off += sizeof(uint16_t) * (size_t)D * (kKeyBlock + 8);
    m.Pk = off;   off += sizeof(uint16_t) * (size_t)kKeyBlock * (F + 8);
    m.rowK = off; off += sizeof(void*) * 2 * kKeyBlock;  // K row addresses of two key blocks
    m.rowV = off; off += sizeof(void*) * 2 * kKeyBlock;
    m.refs = off; off += align_up(sizeof(int) * (size_t)(C > 0 ? C : 1), 16);
    m.total = align_up(off, 16);
    return m;
}

// position of key k (0..31) of a 32-key step in the P^T / V^T operand order
__device__ __forceinline__ int key_perm(int k) { return ((k & 15) >> 2) * 8 + (k >> 4) * 4 + (k & 3); }

template <int D, int F>
__global__ __launch_bounds__(kOutThreads) void output_kernel_bf16(Args a)
{
    constexpr int NT = kOutThreads, NW = NT / 64, RT = 2, KB = kKeyBlock, Fh = F / 2, FM = F / 32, DS = D / 32,
                  DT = D / 16;
    constexpr int KP = D + 8, VP = KB + 8, PP = F + 8;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    if (!state_ok(a)) return;  // header mismatch or faulted state: nothing is read or written
    const Dims& d = a.d;
    constexpr OutSmem sm = out_smem<D, F>(1);  // every offset used here is independent of C
    float* sP = (float*)(smem + sm.sP);
    int* srefL = (int*)(smem + sm.refs);
    uint16_t* Ks = (uint16_t*)(smem + sm.Ks);
    uint16_t* VT = (uint16_t*)(smem + sm.VT);
    uint16_t* Pk = (uint16_t*)(smem + sm.Pk);
    uint16_t* Wl = (uint16_t*)(smem + sm.Wl);
    uint16_t* Hs = (uint16_t*)(smem + sm.Hs);
    const bf16** rowK = (const bf16**)(smem + sm.rowK);
    const bf16** rowV = (const bf16**)(smem + sm.rowV);

    const int G = d.G, L = d.L, w = d.w;
    const int chain = blockIdx.y, b = chain / d.Hkv, g = chain % d.Hkv;
    const int rows = G * L;
    const int wpi = (rows + kOutRows - 1) / kOutRows;
    const int c = blockIdx.x / wpi, rblk = blockIdx.x % wpi;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, qg = lane >> 4;
    const int NI = a.NI;
    const int ns = seq_tokens(a, b);
    if ((int64_t)c * L >= ns) return;  // past this sequence's tokens (the whole workgroup)
    const int64_t t0 = ws_t0(a, b);
    const int64_t ap = t0 + (int64_t)c * L;
    const int64_t ep = ap + L < t0 + ns ? ap + L : t0 + ns;
    const int Lc = (int)(ep - ap);

    // ---- stage s_c (operand order) and the cache refs of the snapshot ----
    const uint16_t* HTg = (const uint16_t*)(a.ws + a.wl.snapH) + ((size_t)chain * NI + c) * F * D;  // [D][F] bf16
    const uint16_t* Whg = (const uint16_t*)(a.state + a.sl.Wb) + (size_t)(3 * g) * Fh * D;          // [Fh][D]
    {
        constexpr int WN = 2 * Fh * D / 8 / NT, HN = D * F / 8 / NT;  // 16-byte pieces per thread
        uint4 w4[WN], h4[HN];
#pragma unroll
        for (int k = 0; k < WN; ++k) w4[k] = *(const uint4*)(Whg + (size_t)(tid + k * NT) * 8);
#pragma unroll
        for (int k = 0; k < HN; ++k) h4[k] = *(const uint4*)(HTg + (size_t)(tid + k * NT) * 8);
#pragma unroll
        for (int k = 0; k < WN; ++k) {
            const int e = (tid + k * NT) * 8;  // row = part * Fh + feature
            *(uint4*)(Wl + (e / D) * (D + 8) + e % D) = w4[k];
        }
#pragma unroll
        for (int k = 0; k < HN; ++k) {
            const int e = (tid + k * NT) * 8;
            *(uint4*)(Hs + (e / F) * (F + 8) + e % F) = h4[k];
        }
        const float* sS = (const float*)(a.ws + a.wl.snapS) + ((size_t)chain * NI + c) * F;
        for (int i = tid; i < F; i += NT) sP[perm_pos(i)] = sS[i];
        const int Cp0 = d.C > 0 ? d.C : 1;
        const int cc0 = ((const int*)(a.ws + a.wl.snapN))[(size_t)chain * NI + c];
        const int* sr0 = (const int*)(a.ws + a.wl.snapRef) + ((size_t)chain * NI + c) * Cp0;
        for (int i = tid; i < cc0; i += NT) srefL[i] = sr0[i];
    }

    // ---- this lane's queries (columns r16 of the wave's two row tiles) ----
    int64_t tq[RT];
    int hq_[RT];
    bool qv[RT];
    bf16x8 qf[RT][DS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = rblk * kOutRows + wave * (16 * RT) + rt * 16 + r16;
        const int hl = r / L, ti = r % L;
        qv[rt] = r < rows && ti < Lc;
        hq_[rt] = g * G + (qv[rt] ? hl : 0);
        tq[rt] = qv[rt] ? ap + ti : -1;
        const bf16* qp = (const bf16*)a.q + (((size_t)b * a.n + (size_t)(qv[rt] ? ap + ti - t0 : 0)) * d.Hq + hq_[rt]) * D;
#pragma unroll
        for (int ks = 0; ks < DS; ++ks) {
            const uint4 u4 = qv[rt] ? *(const uint4*)(qp + ks * 32 + qg * 8) : make_uint4(0, 0, 0, 0);
            qf[rt][ks] = __builtin_bit_cast(bf16x8, u4);
        }
    }
    __syncthreads();

    // ---- keys: window span [sp0, ep) then the snapshot cache ----
    const int Cp = d.C > 0 ? d.C : 1;
    const int64_t sp0 = ap - w > 0 ? ap - w : 0;
    const int nSpan = (int)(ep - sp0);
    const int ccnt = ((const int*)(a.ws + a.wl.snapN))[(size_t)chain * NI + c];
    const int* sref = srefL;
    const int nK = nSpan + ccnt;
    const int xs0 = (int)(sp0 - (t0 - w));
    const float tau = d.tau;
    const int64_t lastPend = ep - 1 - w;
    constexpr int KU = (KB * D / 8 + NT - 1) / NT;  // 16-byte units per thread for K
    constexpr int PU = (KB * F / 8 + NT - 1) / NT;  // for phi(K)
    constexpr int VPU = (KB / 2) * (D / 8);         // (key pair, 8-value unit) items for V
    static_assert(VPU <= NT, "one V key-pair unit per thread at most");
    uint4 pk[KU], pv[2], pp[PU];
    // Row addresses of the KB keys of block j go to table j % 2, written by one
    // wave two blocks ahead of the prefetch that reads them.
    auto fill_rows = [&](int j, int i) {
        const int kidx = j * KB + i, kc = kidx < nK ? kidx : 0;
        const int ref = kc < nSpan ? xs0 + kc : sref[kc - nSpan];
        rowK[(j & 1) * KB + i] = ref_k<bf16>(a, chain, b, g, ref);
        rowV[(j & 1) * KB + i] = ref_v<bf16>(a, chain, b, g, ref);
    };
#define LOLA_OUT_PREFETCH(BASE, PHI)                                                                                 \
    do {                                                                                                             \
        const int tb = (((BASE) / KB) & 1) * KB;                                                                     \
        _Pragma("unroll") for (int k = 0; k < KU; ++k) {                                                             \
            const int idx = tid + k * NT, kr = (idx / (D / 8)) % KB, un = idx % (D / 8);                             \
            const uint4 k4 = *(const uint4*)(rowK[tb + kr] + un * 8);                                                \
            pk[k] = (BASE) + kr < nK ? k4 : make_uint4(0, 0, 0, 0);                                                  \
        }                                                                                                            \
        if (tid < VPU) {                                                                                             \
            const int pr = tid % (KB / 2), un = tid / (KB / 2);                                                      \
            _Pragma("unroll") for (int k = 0; k < 2; ++k) {                                                          \
                const uint4 v4 = *(const uint4*)(rowV[tb + 2 * pr + k] + un * 8);                                   \
                pv[k] = (BASE) + 2 * pr + k < nK ? v4 : make_uint4(0, 0, 0, 0);                                      \
            }                                                                                                        \
        }                                                                                                            \
        if (PHI) _Pragma("unroll") for (int k = 0; k < PU; ++k) {                                                    \
            const int idx = tid + k * NT, kr = (idx / (F / 8)) % KB, un = idx % (F / 8), kidx = (BASE) + kr;         \
            const bool want = kidx < nSpan && sp0 + kidx <= lastPend;                                                \
            const uint4 p4 = *(const uint4*)(ws_phiS(a, chain, xs0 + (want ? kidx : 0)) + un * 8);                   \
            pp[k] = want ? p4 : make_uint4(0, 0, 0, 0);                                                              \
        }                                                                                                            \
    } while (0)
    if (tid < 2 * KB) fill_rows(tid / KB, tid % KB);
    __syncthreads();  // tables of blocks 0 and 1
    if (nK > 0) LOLA_OUT_PREFETCH(0, true);  // in flight while phi(q) and the linear read run

    // ---- phi(q): z^T = W Q^T (W hi + lo), two softmax halves per query ----
    bf16x8 pf[RT][FM];
    float zl[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        floatx4 zt[Fh / 16];
#pragma unroll
        for (int ft = 0; ft < Fh / 16; ++ft) {
            zt[ft] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DS; ++ks) {
                const int o = (ft * 16 + r16) * (D + 8) + ks * 32 + qg * 8;
                zt[ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(Wl + o), qf[rt][ks], zt[ft], 0, 0, 0);
                zt[ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(Wl + Fh * (D + 8) + o), qf[rt][ks], zt[ft], 0, 0, 0);
            }
        }
        float zmax = -INFINITY, zmin = INFINITY;
#pragma unroll
        for (int ft = 0; ft < Fh / 16; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) { zmax = fmaxf(zmax, zt[ft][i]); zmin = fminf(zmin, zt[ft][i]); }
        zmax = quad_max(zmax);
        zmin = quad_min(zmin);
        float ph[Fh / 4], pn[Fh / 4];
        float sp = 0.f, sn = 0.f;
#pragma unroll
        for (int ft = 0; ft < Fh / 16; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ph[ft * 4 + i] = __expf(zt[ft][i] - zmax);
                pn[ft * 4 + i] = __expf(zmin - zt[ft][i]);
                sp += ph[ft * 4 + i];
                sn += pn[ft * 4 + i];
            }
        sp = quad_sum(sp);
        sn = quad_sum(sn);
        const float isp = 1.f / sp, isn = 1.f / sn;
        // operand order: step mf covers feature tiles 2mf, 2mf+1; features ft*16+qg*4+i
        float hv[F / 4];
#pragma unroll
        for (int ft = 0; ft < Fh / 16; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hv[(ft >> 1) * 8 + (ft & 1) * 4 + i] = ph[ft * 4 + i] * isp;                 // feature ft*16+qg*4+i
                hv[Fh / 4 + (ft >> 1) * 8 + (ft & 1) * 4 + i] = pn[ft * 4 + i] * isn;        // feature Fh+ft*16+...
            }
        float z = 0.f;
#pragma unroll
        for (int mf = 0; mf < FM; ++mf) {
            u16x8 u;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                u[j] = bf16_bits(hv[mf * 8 + j]);
                z += hv[mf * 8 + j] * sP[mf * 32 + qg * 8 + j];
            }
            pf[rt][mf] = __builtin_bit_cast(bf16x8, u);
        }
        z = quad_sum(z);
        zl[rt] = z;
    }

    // ---- linear read of the snapshot state: O^T = H_c^T phi(q)^T ----
    floatx4 O[RT][DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) O[rt][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mf = 0; mf < FM; ++mf) {
            const bf16x8 ha = *(const bf16x8*)(Hs + (dt * 16 + r16) * (F + 8) + mf * 32 + qg * 8);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) O[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ha, pf[rt][mf], O[rt][dt], 0, 0, 0);
        }
    }
    float Zp[RT], mrun[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) { Zp[rt] = qg == 0 ? zl[rt] : 0.f; mrun[rt] = 0.f; }

    // blocks that hold window-span keys (window, linear and masked keys)
    int base = 0;
    for (; base < nK && base < nSpan; base += KB) {
        __syncthreads();  // the previous block and the table of block base / KB are no longer read
        if (tid < KB && base + 2 * KB < nK) fill_rows(base / KB + 2, tid);
#pragma unroll
        for (int k = 0; k < KU; ++k) {
            const int idx = tid + k * NT, kr = idx / (D / 8), un = idx % (D / 8);
            if (idx < KB * D / 8) *(uint4*)(Ks + kr * KP + un * 8) = pk[k];
        }
        if (tid < VPU) {
            // keys 2pr, 2pr+1 sit next to each other in the operand order of their half.
            // A wave covers 32 key pairs x 2 value units: its lanes write one row at a
            // time into distinct dwords (units 8 rows apart would share an LDS bank).
            const int pr = tid % (KB / 2), un = tid / (KB / 2), kc = (2 * pr / 32) * 32 + key_perm((2 * pr) % 32);
            const uint32_t w0[4] = {pv[0].x, pv[0].y, pv[0].z, pv[0].w}, w1[4] = {pv[1].x, pv[1].y, pv[1].z, pv[1].w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t lo = (w0[j >> 1] >> (16 * (j & 1))) & 0xffffu;
                const uint32_t hi = (w1[j >> 1] >> (16 * (j & 1))) & 0xffffu;
                *(uint32_t*)(VT + (un * 8 + j) * VP + kc) = lo | (hi << 16);
            }
        }
#pragma unroll
        for (int k = 0; k < PU; ++k) {
            const int idx = tid + k * NT, kr = idx / (F / 8), un = idx % (F / 8);
            if (idx < KB * F / 8) *(uint4*)(Pk + kr * PP + un * 8) = pp[k];
        }
        __syncthreads();
        if (base + KB < nK) LOLA_OUT_PREFETCH(base + KB, true);
#pragma unroll
        for (int st = 0; st < KB / kKeyStep; ++st) {
            const int sb = base + st * kKeyStep;  // first key of this step
            if (sb >= nK) break;                  // (uniform)
            const bool anyPend = sb < nSpan && sp0 + sb <= lastPend;
            constexpr int KT = kKeyStep / 16;  // key tiles per step
            floatx4 sT[RT][KT], kT[RT][KT];
#pragma unroll
            for (int tt = 0; tt < KT; ++tt) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) sT[rt][tt] = kT[rt][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
                const int kr = st * kKeyStep + tt * 16 + r16;  // staged row of this lane's key
#pragma unroll
                for (int ks = 0; ks < DS; ++ks) {
                    const bf16x8 ka = *(const bf16x8*)(Ks + kr * KP + ks * 32 + qg * 8);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) sT[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[rt][ks], sT[rt][tt], 0, 0, 0);
                }
                if (anyPend) {
#pragma unroll
                    for (int mf = 0; mf < FM; ++mf) {
                        const bf16x8 pa = *(const bf16x8*)(Pk + kr * PP + mf * 32 + qg * 8);
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) kT[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, pf[rt][mf], kT[rt][tt], 0, 0, 0);
                    }
                }
            }
            bf16x8 pb[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                // the lane's 8 keys: sb + tt*16 + qg*4 + i (tt = j / 4, i = j % 4); key j
                // sits in slot j of the P^T operand
                constexpr int NJ = kKeyStep / 4;
                float lg[NJ];
                int kind[NJ];
                float bmax = -INFINITY;
                // query position relative to the span start; span key kidx sits at sp0 + kidx
                const int tr = qv[rt] ? (int)(tq[rt] - sp0) : -1;
                // kind 1: softmax key (in the query's window, or a cache key), 2: linear key
                // (left the window inside the interval, before the query), 0: masked; all
                // selects, no branches
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int tt = j >> 2, i = j & 3;
                    const int kidx = sb + tt * 16 + qg * 4 + i;
                    const int kspan = kidx <= tr ? (kidx >= tr - w + 1 ? 1 : 2) : 0;
                    kind[j] = (tr >= 0 && kidx < nK) ? (kidx < nSpan ? kspan : 1) : 0;
                    lg[j] = tau * sT[rt][tt][i];
                    bmax = fmaxf(bmax, kind[j] == 1 ? lg[j] : -INFINITY);
                }
                bmax = quad_max(bmax);
                // the reference moves only when a logit exceeds it by more than kRescaleGap
                // (for the whole wave); weights stay below e^kRescaleGap, o = O / Z is unchanged
                if (__builtin_amdgcn_ballot_w64(bmax > mrun[rt] + kRescaleGap) != 0ull) {
                    const float mnew = fmaxf(mrun[rt], bmax);
                    const float resc = __expf(mrun[rt] - mnew);
                    mrun[rt] = mnew;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) O[rt][dt] *= resc;
                    Zp[rt] *= resc;
                }
                const float mnew = mrun[rt];
                const float elin = __expf(-mnew);
                u16x8 u;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int tt = j >> 2, i = j & 3;
                    const float e1 = __expf(lg[j] - mnew), e2 = kT[rt][tt][i] * elin;
                    const float pv_ = kind[j] == 1 ? e1 : (kind[j] == 2 ? e2 : 0.f);
                    Zp[rt] += pv_;
                    u[j] = bf16_bits(pv_);
                }
                pb[rt] = __builtin_bit_cast(bf16x8, u);
            }
            // O^T += V^T P^T
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 va = *(const bf16x8*)(VT + (dt * 16 + r16) * VP + st * kKeyStep + qg * 8);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    O[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rt], O[rt][dt], 0, 0, 0);
            }
        }
    }

    // Blocks past the window span hold cache keys only (and, in the last block, slots
    // past the count, masked): no linear keys, so no phi(K) rows, no kappa and no
    // classification.  The softmax reference m of a row moves only when a logit exceeds
    // it by more than kRescaleGap (decided for the whole wave), so O and Z are rarely
    // rescaled; weights e^(logit - m) stay below e^kRescaleGap, and any m gives the same
    // o = O / Z.
    for (; base < nK; base += KB) {
        __syncthreads();  // the previous block and the table of block base / KB are no longer read
        if (tid < KB && base + 2 * KB < nK) fill_rows(base / KB + 2, tid);
#pragma unroll
        for (int k = 0; k < KU; ++k) {
            const int idx = tid + k * NT, kr = idx / (D / 8), un = idx % (D / 8);
            if (idx < KB * D / 8) *(uint4*)(Ks + kr * KP + un * 8) = pk[k];
        }
        if (tid < VPU) {
            const int pr = tid % (KB / 2), un = tid / (KB / 2), kc = (2 * pr / 32) * 32 + key_perm((2 * pr) % 32);
            const uint32_t w0[4] = {pv[0].x, pv[0].y, pv[0].z, pv[0].w}, w1[4] = {pv[1].x, pv[1].y, pv[1].z, pv[1].w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t lo = (w0[j >> 1] >> (16 * (j & 1))) & 0xffffu;
                const uint32_t hi = (w1[j >> 1] >> (16 * (j & 1))) & 0xffffu;
                *(uint32_t*)(VT + (un * 8 + j) * VP + kc) = lo | (hi << 16);
            }
        }
        __syncthreads();
        if (base + KB < nK) LOLA_OUT_PREFETCH(base + KB, false);
#pragma unroll
        for (int st = 0; st < KB / kKeyStep; ++st) {
            const int sb = base + st * kKeyStep;  // first key of this step
            if (sb >= nK) break;                  // (uniform)
            constexpr int KT = kKeyStep / 16;
            floatx4 sT[RT][KT];
#pragma unroll
            for (int tt = 0; tt < KT; ++tt) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) sT[rt][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
                const int kr = st * kKeyStep + tt * 16 + r16;
#pragma unroll
                for (int ks = 0; ks < DS; ++ks) {
                    const bf16x8 ka = *(const bf16x8*)(Ks + kr * KP + ks * 32 + qg * 8);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) sT[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[rt][ks], sT[rt][tt], 0, 0, 0);
                }
            }
            bf16x8 pb[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                // the lane's 8 keys: sb + tt*16 + qg*4 + i (tt = j / 4, i = j % 4), slot j of P^T
                constexpr int NJ = kKeyStep / 4;
                float lg[NJ];
                float bmax = -INFINITY;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int kidx = sb + (j >> 2) * 16 + qg * 4 + (j & 3);
                    lg[j] = kidx < nK ? tau * sT[rt][j >> 2][j & 3] : -INFINITY;
                    bmax = fmaxf(bmax, lg[j]);
                }
                bmax = quad_max(bmax);
                if (__builtin_amdgcn_ballot_w64(bmax > mrun[rt] + kRescaleGap) != 0ull) {
                    const float mnew = fmaxf(mrun[rt], bmax);
                    const float resc = __expf(mrun[rt] - mnew);
                    mrun[rt] = mnew;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) O[rt][dt] *= resc;
                    Zp[rt] *= resc;
                }
                u16x8 u;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const float e1 = __expf(lg[j] - mrun[rt]);  // 0 for a masked slot
                    Zp[rt] += e1;
                    u[j] = bf16_bits(e1);
                }
                pb[rt] = __builtin_bit_cast(bf16x8, u);
            }
            // O^T += V^T P^T
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 va = *(const bf16x8*)(VT + (dt * 16 + r16) * VP + st * kKeyStep + qg * 8);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    O[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rt], O[rt][dt], 0, 0, 0);
            }
        }
    }

#undef LOLA_OUT_PREFETCH
    // ---- shared denominator, store o[t][h][d] ----
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        float Z = Zp[rt];
        Z = quad_sum(Z);
        if (qv[rt]) {
            bf16* op = (bf16*)a.out + (((size_t)b * a.n + (size_t)(tq[rt] - t0)) * d.Hq + hq_[rt]) * D;
            const float inv = 1.f / Z;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const uint32_t lo = (uint32_t)bf16_bits(O[rt][dt][0] * inv) | ((uint32_t)bf16_bits(O[rt][dt][1] * inv) << 16);
                const uint32_t hi = (uint32_t)bf16_bits(O[rt][dt][2] * inv) | ((uint32_t)bf16_bits(O[rt][dt][3] * inv) << 16);
                *(uint2*)(op + dt * 16 + qg * 4) = make_uint2(lo, hi);
            }
        }
    }
}

}  // namespace lola
