// Decode step for bf16 io (gfx950): one one-token update interval per
// (sequence, KV head) chain, one workgroup (4 waves) per chain, state read and
// written in place.
//
//   read   -- the chain's G query heads (MFMA columns) attend with exact
//             softmax to the window [t-w+1, t] and the cache, streamed in
//             blocks of 128 keys (32 per wave) with an online softmax per wave,
//             merged at the end; the linear part is H^T phi(q) / s . phi(q)
//             plus the key at t-w that leaves the window at this step (the new
//             key itself when w = 0); one shared denominator (LoLA summary,
//             "Inferentiestrategie", step 4).
//   manage -- the SRE equation ("Het Self-Recall Error (SRE) Mechanisme") for
//             every cached key and the leaving key against the step-start
//             state: the cached keys' features come from their stored bf16
//             hi/lo rows (written when each key entered the cache), the
//             leaving key's are computed, phi(k) = [softmax(W k); softmax(-W k)]
//             by MFMA with W in three bf16 parts; n^T = H^T phi^T with H and
//             phi in bf16 hi/lo parts, d = phi . s; then the pair with the
//             lowest SRE (newest on a tie) is folded into H, s by one outer
//             product when the candidates exceed the capacity, and the leaving
//             key takes its cache slot with its feature row.
#pragma once

#include <type_traits>

#include "lola_output.h"

namespace lola {

constexpr int kDecBlock = 128;  // keys staged per block (32 per wave)

struct DecSmem {
    size_t HhT, HlT, Wl, sP, cposL, esc, phiE, phiF, xrow, stVT, misc, total;
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
    m.phiE = off;  off += align_up(sizeof(float) * F, 16);
    m.phiF = off;  off += align_up(sizeof(float) * F, 16);
    m.xrow = off;  off += align_up(sizeof(float) * D, 16);
    m.stVT = off;  off += align_up(sizeof(uint16_t) * (size_t)D * (kDecBlock + 8), 16);
    m.misc = off;  off += align_up(sizeof(int) * 16, 16);
    m.cposL = off; off += align_up(sizeof(int) * (size_t)Cp, 16);
    m.esc = off;   off += align_up(sizeof(float) * (size_t)(Cp + 1), 16);
    m.total = align_up(off, 16);
    return m;
}

// e^x as 2^(x log2 e): the product is carried in two floats (log2 e split into
// a float and its remainder, as in Cody and Waite's argument reduction), so the
// hardware 2^ instruction sees an argument good to about 2^-40 relative and
// 2^r = 1 + r ln 2 covers the small remainder r.  Arguments here are <= 0.
__device__ __forceinline__ float exp_acc(float x)
{
    constexpr float kL1 = 1.44269502162933349609375f;  // log2(e) rounded to float
    constexpr float kL2 = 1.9259629911783447e-08f;     // log2(e) - kL1
    const float t = x * kL1;
    const float r = fmaf(x, kL1, -t) + x * kL2;
    return __builtin_amdgcn_exp2f(t) * fmaf(r, 0.693147180559945309f, 1.0f);
}

// phi = [softmax(W k); softmax(-W k)] of P tiles of 16 keys (key r16 of tile p in
// column r16 of kb[p]): z^T = W K^T by MFMA with W in three bf16 parts (exact
// products against bf16 keys, fp32 sums; the W operands are read once for all P
// tiles), then one softmax per half over the features.  x[p][h] is the feature
// of operand slot h: slot h = 8 mf + j holds feature 16 (2 mf + j / 4) + 4 qg + j % 4
// (positive half for mf < F / 64).
template <int D, int F, int P>
__device__ __forceinline__ void phi_tiles(const uint16_t* Wl, const bf16x8 (*kb)[D / 32], int r16, int qg,
                                          float (*x)[F / 4])
{
    constexpr int Fh = F / 2, DS = D / 32, WS = D + 8;  // Wl: [3][Fh][WS] in LDS
    floatx4 zt[P][Fh / 16];
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

// feature index of operand slot h (see phi_tile) for lane group qg
__device__ __forceinline__ int slot_feature(int h, int qg) { return (2 * (h >> 3) + ((h & 7) >> 2)) * 16 + qg * 4 + (h & 3); }

template <int D, int F>
__global__ __launch_bounds__(256, 1) void decode_kernel_bf16(Args a)
{
    constexpr int NW = 4, Fh = F / 2, FM = F / 32, DS = D / 32, DT = D / 16;
    constexpr int KBL = kDecBlock, KW = KBL / NW;  // keys per block, per wave
    constexpr int HP = F + 8, VP = KBL + 8;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const Dims& d = a.d;
    const int G = d.G, w = d.w, C = d.C;
    const DecSmem sm = dec_smem<D, F>(C);  // only the last two offsets depend on C
    uint16_t* HhT = (uint16_t*)(smem + sm.HhT);
    uint16_t* HlT = (uint16_t*)(smem + sm.HlT);
    float* sP = (float*)(smem + sm.sP);
    int* cposL = (int*)(smem + sm.cposL);
    float* esc = (float*)(smem + sm.esc);
    float* phiE = (float*)(smem + sm.phiE);
    float* phiF = (float*)(smem + sm.phiF);
    float* xrow = (float*)(smem + sm.xrow);
    uint16_t* Wl = (uint16_t*)(smem + sm.Wl);
    uint16_t* stVT = (uint16_t*)(smem + sm.stVT);
    int* misc = (int*)(smem + sm.misc);
    float* mrg = (float*)(smem + sm.stVT);  // merge area, reused after the key loop

    const int chain = blockIdx.x, b = chain / d.Hkv, g = chain % d.Hkv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, qg = lane >> 4;
    Chain ch = chain_of(a, chain);
    const int64_t t = ch.tok();
    const int cnt = min(max(ch.cnt(), 0), C);
    const bf16* knew = (const bf16*)a.k + ((size_t)b * d.Hkv + g) * D;
    const bf16* vnew = (const bf16*)a.v + ((size_t)b * d.Hkv + g) * D;
    const bool hasE = (w == 0) || (t - w >= 0);
    const int64_t pE = t - w;
    const int rs = w > 0 ? (int)(t % w) : 0;
    const bf16* kE = w == 0 ? knew : ch.ring_k<bf16>() + (size_t)rs * D;
    const bf16* vE = w == 0 ? vnew : ch.ring_v<bf16>() + (size_t)rs * D;
    const uint16_t* Wb = (const uint16_t*)(a.state + a.sl.Wb) + (size_t)(3 * g) * Fh * D;

    // ---- state in: H^T hi/lo in operand order, s, cache positions ----
    {
        const float* Hst = ch.H();  // [D][F]
        constexpr int HN = D * F / 4 / 256;  // float4 per thread, all loaded before any is used
        constexpr int WN = 3 * Fh * D / 8 / 256;  // 16-byte pieces of the W parts per thread
        // W parts to LDS in batches of WB pieces (all loads of a batch issued before
        // any is stored; larger batches would need more registers than the wave has)
        constexpr int WB = WN % 4 == 0 ? 4 : (WN % 3 == 0 ? 3 : 1);
        // H (from HBM, the longest wait) is requested first, all of it; the W batches
        // (L2 hits) are stored to LDS while it is in flight
        float4 hv4[HN];
#pragma unroll
        for (int k = 0; k < HN; ++k) hv4[k] = *(const float4*)(Hst + (size_t)(tid + k * 256) * 4);
#pragma unroll
        for (int k0 = 0; k0 < WN; k0 += WB) {
            uint4 w4[WB];
#pragma unroll
            for (int k = 0; k < WB; ++k) w4[k] = *(const uint4*)(Wb + (size_t)(tid + (k0 + k) * 256) * 8);
#pragma unroll
            for (int k = 0; k < WB; ++k) {
                const int e = (tid + (k0 + k) * 256) * 8, row = e / D, col = e % D;  // row = part * Fh + feature
                *(uint4*)(Wl + row * (D + 8) + col) = w4[k];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int k = 0; k < HN; ++k) {
            const int i = tid + k * 256, dd = (i * 4) / F, f = (i * 4) % F;
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
        for (int i = tid; i < F; i += 256) sP[perm_pos(i)] = ch.s()[i];
        for (int i = tid; i < cnt; i += 256) cposL[i] = ch.cpos()[i];
    }
    // query frags (columns r16 < G); the leaving key's row (wave 3, column 0) and
    // its value rows dt * 16 + 4 qg .. + 3 (waves 0 and 3)
    bf16x8 qf[DS];
    uint4 kEq[DS];
    uint2 vEq[DT];
    {
        const bool le = hasE && (wave == 0 || wave == NW - 1);
#pragma unroll
        for (int ks = 0; ks < DS; ++ks)
            kEq[ks] = (hasE && wave == NW - 1 && r16 == 0) ? *(const uint4*)(kE + ks * 32 + qg * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vEq[dt] = le ? *(const uint2*)(vE + dt * 16 + qg * 4) : make_uint2(0, 0);
        const bool qv = r16 < G;
        const bf16* qp = (const bf16*)a.q + ((size_t)b * d.Hq + g * G + (qv ? r16 : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < DS; ++ks) {
            const uint4 u4 = qv ? *(const uint4*)(qp + ks * 32 + qg * 8) : make_uint4(0, 0, 0, 0);
            qf[ks] = __builtin_bit_cast(bf16x8, u4);
        }
    }
    __syncthreads();  // W parts and H in LDS
    // Error of P tiles of 16 candidates from their feature operands (bf16 hi, lo
    // parts bh, bl; candidate r16 of tile p) and 1 / d: n^T = H^T phi^T with H and phi
    // in hi/lo parts (hi.hi + lo.hi + hi.lo; the H operands are read once for all P
    // tiles), e = |n / d - v|^2 (values vq[p] at rows dt * 16 + 4 qg .. + 3, cv[p]
    // whether the column is a candidate)
    auto sre_core = [&](auto pTag, const bf16x8 (*bh)[FM], const bf16x8 (*bl)[FM], const float* inv, const bool* cv,
                        const uint2 (*vq)[DT], float* e) {
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
                const float vv[4] = {__uint_as_float(vq[p][dt].x << 16), __uint_as_float(vq[p][dt].x & 0xffff0000u),
                                     __uint_as_float(vq[p][dt].y << 16), __uint_as_float(vq[p][dt].y & 0xffff0000u)};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float df = (acc[p][i] + acc2[p][i]) * inv[p] - (cv[p] ? vv[i] : 0.f);
                    es[p] += df * df;
                }
            }
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            es[p] = quad_sum(es[p]);
            e[p] = es[p];
        }
    };
    // 1 / d with d = s . (phi hi + phi lo): the feature values the MFMAs see (the
    // prefill scan scores with the same 16-bit features)
    auto inv_d = [&](const bf16x8* bh, const bf16x8* bl) -> float {
        float dd = 0.f;
#pragma unroll
        for (int mf = 0; mf < FM; ++mf) {
            const u16x8 uh = __builtin_bit_cast(u16x8, bh[mf]), ul = __builtin_bit_cast(u16x8, bl[mf]);
#pragma unroll
            for (int j = 0; j < 8; ++j) dd += (bf16_val(uh[j]) + bf16_val(ul[j])) * sP[mf * 32 + qg * 8 + j];
        }
        dd = quad_sum(dd);
        return dd > 0.f ? 1.f / dd : 0.f;
    };
    // SRE of P tiles whose features are computed here from the key fragments kb[p]
    auto sre_tiles = [&](auto pTag, const bf16x8 (*kb)[DS], const bool* cv, const uint2 (*vq)[DT], float* e,
                         float* phi0 = nullptr) {  // phi0: phi of candidate 0 of tile 0, natural order
        constexpr int P = decltype(pTag)::value;
        bf16x8 bh[P][FM], bl[P][FM];
        float inv[P];
        {
            float x[P][F / 4];
            phi_tiles<D, F, P>(Wl, kb, r16, qg, x);
            if (phi0 && r16 == 0)
#pragma unroll
                for (int h = 0; h < F / 4; ++h) phi0[slot_feature(h, qg)] = x[0][h];
#pragma unroll
            for (int p = 0; p < P; ++p) {
#pragma unroll
                for (int mf = 0; mf < FM; ++mf) {
                    u16x8 uh, ul;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float xv = x[p][mf * 8 + j];
                        const uint16_t h = bf16_bits(xv);
                        uh[j] = h;
                        ul[j] = bf16_bits(xv - bf16_val(h));
                    }
                    bh[p][mf] = __builtin_bit_cast(bf16x8, uh);
                    bl[p][mf] = __builtin_bit_cast(bf16x8, ul);
                }
                inv[p] = inv_d(bh[p], bl[p]);
            }
        }
        sre_core(pTag, bh, bl, inv, cv, vq, e);
    };

    // Wave 3: phi of the leaving key (column 0 of a tile) and, when a pair must be
    // folded, its SRE against the step-start state.  Meanwhile wave 0, the only wave
    // that needs phi(q), computes it and the linear read O_lin^T = H^T phi(q)^T; the
    // leaving key's share of the linear part is added once its features are in LDS.
    const int nU = cnt + (hasE ? 1 : 0);
    floatx4 O[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mrun = 0.f, Zp = 0.f;
    float xq[F / 4];  // wave 0: phi(q) of column r16, operand-slot order
    float zq = 0.f;   // wave 0: s . phi(q)
    if (wave == NW - 1) {
        bf16x8 kb[1][DS];
#pragma unroll
        for (int ks = 0; ks < DS; ++ks) kb[0][ks] = __builtin_bit_cast(bf16x8, kEq[ks]);
        if (hasE && nU > C) {
            const bool cv[1] = {r16 == 0};
            uint2 vq[1][DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) vq[0][dt] = vEq[dt];
            float e[1];
            sre_tiles(std::integral_constant<int, 1>{}, kb, cv, vq, e, phiE);
            if (lane == 0) esc[cnt] = e[0];
        } else {
            float x[1][F / 4];
            phi_tiles<D, F, 1>(Wl, kb, r16, qg, x);
            if (r16 == 0)
#pragma unroll
                for (int h = 0; h < F / 4; ++h) phiE[slot_feature(h, qg)] = x[0][h];
        }
    } else if (wave == 0) {
        // phi(q) for the query columns: z^T = W Q^T with W hi + lo
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
    }
    __syncthreads();  // phi of the leaving key in LDS
    if (wave == 0) {
        // the leaving key's linear weight kappa = phi(q) . phi(k_E) per query column;
        // kappa * v_E joins the linear part (weight e^-M, M floored at 0)
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

    // ---- keys: window [ws0, t] then cache slots; blocks of 128, 32 per wave ----
    const int64_t ws0 = t - w + 1 > 0 ? t - w + 1 : 0;
    const int nWin = w > 0 ? (int)(t - ws0 + 1) : 0;
    const int nK = nWin + cnt;
    // row of key kidx (0 <= kidx < nK): window position ws0 + kidx (ring slot
    // (ws0 + kidx) mod w, the newest being this step's token), then cache slot
    // kidx - nWin; chosen by selects so that a block's loads issue together
    const int rs0 = w > 0 ? (int)(ws0 % w) : 0;
    auto key_row = [&](int kidx, bool v) -> const bf16* {
        int slot = rs0 + kidx;
        slot = slot >= w ? slot - w : slot;
        const bf16* pw = (v ? ch.ring_v<bf16>() : ch.ring_k<bf16>()) + (size_t)slot * D;
        const bf16* pc = (v ? ch.cache_v<bf16>() : ch.cache_k<bf16>()) + (ptrdiff_t)(kidx - nWin) * D;
        const bf16* pn = v ? vnew : knew;
        return kidx < nWin ? (kidx == nWin - 1 ? pn : pw) : pc;
    };
    const float tau = d.tau;

    const int nblk = (nK + KBL - 1) / KBL;
    // Block bi + 1's key fragments and value rows load while block bi is scored; rows
    // past nK load the last key and are zeroed.  A wave takes keys base + wave * KW +
    // tt * 16 + r16 as MFMA fragments straight from memory (a lane's 16 bytes are
    // contiguous in the key row).
    constexpr int VN = (KBL / 2) * (D / 8) / 256;
    static_assert((KBL / 2) * (D / 8) % 256 == 0, "V units cover the key block exactly");
    uint4 kq[2][DS], vq0[VN], vq1[VN];
    auto issue = [&](int base) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int kidx = base + wave * KW + tt * 16 + r16;
            const bf16* kr = key_row(kidx < nK ? kidx : nK - 1, false);
#pragma unroll
            for (int ks = 0; ks < DS; ++ks) kq[tt][ks] = *(const uint4*)(kr + ks * 32 + qg * 8);
        }
#pragma unroll
        for (int k = 0; k < VN; ++k) {
            const int idx = tid + k * 256, k0 = base + 2 * (idx % (KBL / 2)), un = idx / (KBL / 2);
            vq0[k] = *(const uint4*)(key_row(k0 < nK ? k0 : nK - 1, true) + un * 8);
            vq1[k] = *(const uint4*)(key_row(k0 + 1 < nK ? k0 + 1 : nK - 1, true) + un * 8);
        }
    };
    if (nK > 0) issue(0);
    for (int bi = 0; bi < nblk; ++bi) {
        const int base = bi * KBL;
        __syncthreads();  // previous block consumed
        uint4 kcur[2][DS];  // this block's fragments (kq is refilled below)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int ks = 0; ks < DS; ++ks) kcur[tt][ks] = kq[tt][ks];
#pragma unroll
        for (int k = 0; k < VN; ++k) {
            // a wave covers 64 key pairs of one value unit: each transposed store puts its
            // lanes on distinct dwords of one row (units 8 rows apart share an LDS bank)
            const int idx = tid + k * 256, pr = idx % (KBL / 2), un = idx / (KBL / 2);
            const int k0 = base + 2 * pr, k1 = k0 + 1;
            const uint4 v0 = k0 < nK ? vq0[k] : make_uint4(0, 0, 0, 0);
            const uint4 v1 = k1 < nK ? vq1[k] : make_uint4(0, 0, 0, 0);
            const int kc = (2 * pr / KW) * KW + key_perm((2 * pr) % KW);
            const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w}, w1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t lo = (w0[j >> 1] >> (16 * (j & 1))) & 0xffffu;
                const uint32_t hi = (w1[j >> 1] >> (16 * (j & 1))) & 0xffffu;
                *(uint32_t*)(stVT + (un * 8 + j) * VP + kc) = lo | (hi << 16);
            }
        }
        if (bi + 1 < nblk) issue(base + KBL);
        lds_sync();  // V^T staged; the next block's loads stay in flight
        // this wave's 32 keys: base + wave*32 + tt*16 + r16
        const int kb0 = base + wave * KW;
        if (kb0 >= nK) continue;
        floatx4 sT[2];
        bf16x8 kfr[2][DS];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            sT[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DS; ++ks) {
                kfr[tt][ks] = __builtin_bit_cast(bf16x8, kb0 + tt * 16 + r16 < nK ? kcur[tt][ks] : make_uint4(0, 0, 0, 0));
                sT[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfr[tt][ks], qf[ks], sT[tt], 0, 0, 0);
            }
        }
        // online softmax for the query column r16 over the lane's 8 keys
        {
            float lg[8];
            bool ok[8];
            float bmax = -INFINITY;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int tt = j >> 2, i = j & 3;
                const int kidx = kb0 + tt * 16 + qg * 4 + i;
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
    }

    const bool scoreCache = hasE && nU > C;  // the SRE pass over the cache runs
    const int nT = (cnt + 15) / 16;
    // features of the cached keys come from the state (hi | lo rows in operand order)
    uint4 fq[2][2 * FM];
    uint2 vq[2][DT];
    auto tile_load = [&](int p, int tt) {
        const int slot = tt * 16 + r16 < cnt ? tt * 16 + r16 : cnt - 1;
        const uint16_t* pr = ch.cphi() + (size_t)slot * 2 * F + qg * 8;
        const bf16* vr = ch.cache_v<bf16>() + (size_t)slot * D;
#pragma unroll
        for (int mf = 0; mf < FM; ++mf) {
            fq[p][mf] = *(const uint4*)(pr + mf * 32);
            fq[p][FM + mf] = *(const uint4*)(pr + F + mf * 32);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vq[p][dt] = *(const uint2*)(vr + dt * 16 + qg * 4);
    };
    // the wave's tiles wave, wave + NW, ... two at a time; the first two load while
    // the attention parts are merged, the next two while the current two are scored
    if (scoreCache && wave < nT) tile_load(0, wave);
    if (scoreCache && wave + NW < nT) tile_load(1, wave + NW);

    // ---- merge the waves' softmax parts, add the linear part, store ----
    // (LDS-only barriers: the first cache tiles' loads stay in flight)
    lds_sync();  // staging area becomes the merge area
    {
        float* mM = mrg;                 // [NW][16]
        float* mZ = mrg + NW * 16;       // [NW][16]
        float* mO = mrg + 2 * NW * 16;   // [NW][D][16]
        float Z = Zp;
        Z = quad_sum(Z);
        if (qg == 0) { mM[wave * 16 + r16] = mrun; mZ[wave * 16 + r16] = Z; }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mO[(wave * D + dt * 16 + qg * 4 + i) * 16 + r16] = O[dt][i];
        lds_sync();
        for (int idx = tid; idx < G * D; idx += 256) {
            const int col = idx / D, dd = idx % D;
            float M = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, mM[ww * 16 + col]);
            float num = 0.f, den = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                const float sc = __expf(mM[ww * 16 + col] - M);
                num += sc * mO[(ww * D + dd) * 16 + col];
                den += sc * mZ[ww * 16 + col];
            }
            ((bf16*)a.out)[((size_t)b * d.Hq + g * G + col) * D + dd] = from_f32<bf16>(num / den);
        }
    }

    // ---- SRE of the cached pairs (only when a pair must be folded; the leaving
    //      pair's was scored with its phi): the cache in tiles of 16 slots dealt to
    //      the waves in turn; each tile's key and value rows are loaded while the
    //      previous tiles are scored ----
    if (hasE && nU > C) {
        for (int t0 = wave; t0 < nT; t0 += 2 * NW) {
            const int tl[2] = {t0, t0 + NW};
            bf16x8 bh[2][FM], bl[2][FM];
            float inv[2];
            bool cv[2];
            uint2 vv[2][DT];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                cv[p] = tl[p] * 16 + r16 < cnt;
#pragma unroll
                for (int mf = 0; mf < FM; ++mf) {
                    bh[p][mf] = __builtin_bit_cast(bf16x8, cv[p] ? fq[p][mf] : make_uint4(0, 0, 0, 0));
                    bl[p][mf] = __builtin_bit_cast(bf16x8, cv[p] ? fq[p][FM + mf] : make_uint4(0, 0, 0, 0));
                }
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) vv[p][dt] = vq[p][dt];
            }
            if (t0 + 2 * NW < nT) tile_load(0, t0 + 2 * NW);
            if (t0 + 3 * NW < nT) tile_load(1, t0 + 3 * NW);
#pragma unroll
            for (int p = 0; p < 2; ++p) inv[p] = inv_d(bh[p], bl[p]);
            float e[2];
            if (tl[1] < nT) sre_core(std::integral_constant<int, 2>{}, bh, bl, inv, cv, vv, e);  // wave-uniform
            else sre_core(std::integral_constant<int, 1>{}, bh, bl, inv, cv, vv, e);
#pragma unroll
            for (int p = 0; p < 2; ++p)
                if (tl[p] < nT && qg == 0 && cv[p]) esc[tl[p] * 16 + r16] = e[p];
        }
    }
    __syncthreads();
    int victim = -1;
    if (hasE && nU > C) {
        // H (fp32) for the fold is requested before the victim is known
        float* Hd = ch.H();
        constexpr int HN = D * F / 4 / 256;  // float4 per thread
        float4 h4[HN];
#pragma unroll
        for (int k = 0; k < HN; ++k) h4[k] = *(const float4*)(Hd + (size_t)(tid + k * 256) * 4);
        if (wave == 0) {
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
        }
        lds_sync();  // (LDS-only barriers up to the fold: H stays in flight)
        victim = misc[0];
        // phi of the folded key (wave 0, column 0 of a tile) and its value (wave 1),
        // then H += phi v^T, s += phi
        if (wave == 0) {
            // the folded key's features: its stored row (hi + lo), or the leaving key's
            if (victim < cnt) {
                const uint16_t* pr = ch.cphi() + (size_t)victim * 2 * F;
                for (int f = lane; f < F; f += 64) {
                    const int q = perm_pos(f);
                    phiF[f] = bf16_val(pr[q]) + bf16_val(pr[F + q]);
                }
            } else
                for (int f = lane; f < F; f += 64) phiF[f] = phiE[f];
        } else if (wave == 1) {
            const bf16* vr = victim < cnt ? ch.cache_v<bf16>() + (size_t)victim * D : vE;
            for (int j = lane; j < D; j += 64) xrow[j] = to_f32(vr[j]);
        }
        lds_sync();
#pragma unroll
        for (int k = 0; k < HN; ++k) {
            const int i = (tid + k * 256) * 4, dd = i / F, f = i % F;
            const float vv = xrow[dd];
            h4[k].x += vv * phiF[f];
            h4[k].y += vv * phiF[f + 1];
            h4[k].z += vv * phiF[f + 2];
            h4[k].w += vv * phiF[f + 3];
            *(float4*)(Hd + i) = h4[k];
        }
        for (int f = tid; f < F; f += 256) ch.s()[f] += phiF[f];
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
        for (int j = tid; j < D; j += 256) {
            ch.cache_k<bf16>()[(size_t)slot * D + j] = kE[j];
            ch.cache_v<bf16>()[(size_t)slot * D + j] = vE[j];
        }
        uint16_t* pr = ch.cphi() + (size_t)slot * 2 * F;  // its features: hi | lo, operand order
        for (int f = tid; f < F; f += 256) {
            const float x = phiE[f];
            const uint16_t h = bf16_bits(x);
            pr[perm_pos(f)] = h;
            pr[F + perm_pos(f)] = bf16_bits(x - bf16_val(h));
        }
    }
    if (w > 0)
        for (int j = tid; j < D; j += 256) {
            ch.ring_k<bf16>()[(size_t)rs * D + j] = knew[j];
            ch.ring_v<bf16>()[(size_t)rs * D + j] = vnew[j];
        }
    if (tid == 0) {
        if (slot >= 0) ch.cpos()[slot] = (int32_t)pE;
        if (hasE && nU <= C) ch.cnt() = cnt + 1;
        ch.tok() = t + 1;
    }
}

}  // namespace lola
