// Interval scan with each (sequence, KV head) chain spread over D/16
// workgroups (bf16 io).
//
// The scan of one chain is a recurrence over update intervals: the SRE of the
// cached and leaving pairs is scored against the interval-start state, the
// highest C stay, the rest are folded (LoLA technical summary, gist.science,
// sections "Het Self-Recall Error (SRE) Mechanisme" and "Inferentiestrategie").
// With few chains (one sequence, 8 KV heads) one workgroup per chain leaves
// most of the chip idle and puts every step of an interval on one CU.  Here
// workgroup j of a chain owns columns [16j, 16j + 16) of H:
//
//   * its 8 waves split the candidates 16 at a time; each wave computes
//     n = H^T phi(k) for its 16 columns with bf16 MFMAs on hi/lo parts
//     (hi.hi + lo.hi + hi.lo) and d = s . phi(k) with an MFMA whose A rows are
//     the three bf16 parts of s (so d is s in fp32 times phi hi + lo), and
//     writes the partial error sum_{its columns} (n/d - v)^2 to the workspace;
//   * the chain's workgroups meet at a counter in the workspace (agent-scope
//     release / acquire), and every workgroup adds the D/16 partials in the
//     same order, so all of them take the same keep / fold decision;
//   * each workgroup folds the chosen pairs into its own columns only (phi in
//     three bf16 parts, exact products) and updates s, which every workgroup
//     keeps.
//
// Block b runs on XCD b % 8 (round-robin dispatch), so the D/16 workgroups
// of a chain are placed on one XCD and meet in its L2.  The launch is
// cooperative, so all of them are resident together; a wait that does not end
// within a fixed number of polls marks the state as faulted and returns.
#pragma once

#include "lola_prefill.h"

namespace lola {

constexpr int kSplitThreads = 512;  // 8 waves
constexpr int kSplitGroup = 3;      // candidate tiles a wave loads before computing
constexpr uint32_t kSpinLimit = 1u << 22;

struct SplitSmem {
    size_t P, VS, AX, s, ebits, keep, fold, memb, freed, keptE, cref, cpos, hist, ucode, bcnt, misc, total;
};

__host__ __device__ inline SplitSmem split_smem(int F, int C, int L)
{
    SplitSmem m;
    const int U = C + L, Cp = C > 0 ? C : 1, EP = kFoldChunk + 8;
    size_t off = 0;
    m.P = off;     off += align_up(sizeof(uint16_t) * 3 * (size_t)F * EP, 16);  // [3][F][EP]
    m.VS = off;    off += align_up(sizeof(uint16_t) * 16 * (size_t)EP, 16);     // [16][EP]
    m.AX = off;    off += align_up(sizeof(uint16_t) * 2 * 16 * (size_t)(F + 8), 16);
    m.s = off;     off += sizeof(float) * F;
    m.ebits = off; off += sizeof(uint32_t) * U;
    m.keep = off;  off += sizeof(int) * U;
    m.fold = off;  off += sizeof(int) * U;
    m.memb = off;  off += sizeof(int) * U;
    m.freed = off; off += sizeof(int) * Cp;
    m.keptE = off; off += sizeof(int) * (L + 1);
    m.cref = off;  off += sizeof(int) * Cp;
    m.cpos = off;  off += sizeof(int) * Cp;
    m.hist = off;  off += sizeof(int) * kSelBins;
    m.ucode = off; off += sizeof(int) * U;
    m.bcnt = off;  off += sizeof(int) * 4 * ((U + 63) / 64);
    m.misc = off;  off += sizeof(int) * 16;
    m.total = align_up(off, 16);
    return m;
}

// Grid of the split scan: 8 * (D/16) * ceil(chains / 8) blocks.
__host__ __device__ inline int split_blocks(int D, int chains) { return 8 * (D / 16) * ((chains + 7) / 8); }

template <int D, int F>
__global__ __launch_bounds__(kSplitThreads) void scan_split_kernel(Args a)
{
    constexpr int KW = D / 16, NT = kSplitThreads, NW = NT / 64, FT = F / 16, FM = F / 32;
    constexpr int NB = kSelBins, EC = kFoldChunk, EP = EC + 8, AXS = F + 8, GR = kSplitGroup;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const Dims& d = a.d;
    const int w = d.w, C = d.C, L = d.L;
    const int chains = a.B * d.Hkv;
    const int bid = blockIdx.x, xcd = bid & 7, sb = bid >> 3;
    const int jw = sb % KW, chain = (sb / KW) * 8 + xcd;
    if (chain >= chains) return;  // the whole chain is absent: none of its blocks waits
    const int col0 = 16 * jw;
    const SplitSmem sm = split_smem(F, C, L);
    uint16_t* P = (uint16_t*)(smem + sm.P);
    uint16_t* VS = (uint16_t*)(smem + sm.VS);
    uint16_t* AX = (uint16_t*)(smem + sm.AX);  // [2][16][AXS]: hi, lo of H^T rows col0.., operand order
    float* sP = (float*)(smem + sm.s);
    uint32_t* ebits = (uint32_t*)(smem + sm.ebits);
    int* keep = (int*)(smem + sm.keep);
    int* fold = (int*)(smem + sm.fold);
    int* memb = (int*)(smem + sm.memb);
    int* freed = (int*)(smem + sm.freed);
    int* keptE = (int*)(smem + sm.keptE);
    int* cref = (int*)(smem + sm.cref);
    int* cpos = (int*)(smem + sm.cpos);
    int* hist = (int*)(smem + sm.hist);
    int* ucode = (int*)(smem + sm.ucode);
    int* bcnt = (int*)(smem + sm.bcnt);
    int* misc = (int*)(smem + sm.misc);

    const int b = chain / d.Hkv, g = chain % d.Hkv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, qg = lane >> 4;
    Chain ch = chain_of(a, chain);
    const int64_t t0 = ws_t0(a, b);
    const int n = a.n, NI = a.NI;
    const int Cp = C > 0 ? C : 1;
    const int U = C + L;
    uint32_t* xsync = (uint32_t*)(a.ws + a.wl.xsync) + (size_t)chain * 16;
    uint64_t* xe = (uint64_t*)(a.ws + a.wl.xe) + (size_t)chain * 2 * KW * U;

    // ---- state in ----
    const float* Hst = ch.H();  // H^T [D][F]
    floatx4 Hacc = floatx4{0.f, 0.f, 0.f, 0.f};  // wave < FT: H[wave*16 + qg*4 + i][col0 + r16]
    bf16x8 Ah[FM], Al[FM], As[FM];
    {
        float hv[FT][4];
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) load4(Hst + (size_t)(col0 + r16) * F + ft * 16 + qg * 4, hv[ft]);
#pragma unroll
        for (int ft = 0; ft < FT; ++ft)
            if (ft == wave) Hacc = floatx4{hv[ft][0], hv[ft][1], hv[ft][2], hv[ft][3]};
#pragma unroll
        for (int m = 0; m < FM; ++m) {
            u16x8 h, l;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = hv[2 * m + (j >> 2)][j & 3];
                h[j] = bf16_bits(x);
                l[j] = bf16_bits(x - bf16_val(h[j]));
            }
            Ah[m] = __builtin_bit_cast(bf16x8, h);
            Al[m] = __builtin_bit_cast(bf16x8, l);
        }
    }
    // A operand of d: rows 0, 1, 2 are the three bf16 parts of s, the others zero
    auto build_As = [&]() {
#pragma unroll
        for (int m = 0; m < FM; ++m) {
            u16x8 h;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = sP[m * 32 + qg * 8 + j];
                const uint16_t p1 = bf16_bits(x);
                const float r1 = x - bf16_val(p1);
                const uint16_t p2 = bf16_bits(r1);
                const uint16_t p3 = bf16_bits(r1 - bf16_val(p2));
                h[j] = r16 == 0 ? p1 : (r16 == 1 ? p2 : (r16 == 2 ? p3 : (uint16_t)0));
            }
            As[m] = __builtin_bit_cast(bf16x8, h);
        }
    };
    for (int i = tid; i < F; i += NT) sP[perm_pos(i)] = ch.s()[i];
    int cnt = min(max(ch.cnt(), 0), C);
    for (int i = tid; i < cnt; i += NT) {
        cpos[i] = ch.cpos()[i];
        cref[i] = -(i + 1);
    }
    __syncthreads();
    build_As();
    // block 0 rewrites s, the count and the cache positions at the end: it waits
    // until every block of the chain has read them (counter xsync[2])
    if (tid == 0) __hip_atomic_fetch_add(&xsync[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    uint32_t arrivals = 0;  // exchanges this block has completed
    const uint16_t* phiS0 = ws_phiS(a, chain, 0);
    const uint16_t* cphiS0 = ws_cphiS(a, chain, 0);
    const float* phiX0 = ws_phiX(a, chain, 0);
    const float* cphi0 = ws_cphi(a, chain, 0);
    const bf16* vin0 = (const bf16*)a.v + ((size_t)b * n * d.Hkv + g) * D;
    const bf16* ring0v = (const bf16*)(a.ws + a.wl.ring0_v) + (size_t)chain * w * D;
    const bf16* cache0v = (const bf16*)(a.ws + a.wl.cache0_v) + (size_t)chain * Cp * D;
    auto code_phs = [&](int code) -> const uint16_t* {
        return code >= 0 ? phiS0 + (size_t)code * 2 * F : cphiS0 + (size_t)(-code - 1) * 2 * F;
    };
    auto code_phi = [&](int code) -> const float* {
        return code >= 0 ? phiX0 + (size_t)code * F : cphi0 + (size_t)(-code - 1) * F;
    };
    auto code_v = [&](int code) -> const bf16* {
        const bf16* pin = vin0 + (size_t)(code - w) * d.Hkv * D;
        const bf16* pring = ring0v + (size_t)code * D;
        const bf16* pcache = cache0v + (size_t)(-code - 1) * D;
        return code >= w ? pin : (code >= 0 ? pring : pcache);
    };

    for (int c = 0; c < NI; ++c) {
        const int64_t ap = t0 + (int64_t)c * L;
        const int64_t ep = ap + L < t0 + n ? ap + L : t0 + n;

        // ---- interval-start snapshot: H^T hi parts of this block's rows, s and cache refs ----
        if (wave == 0) {
            uint16_t* dst = (uint16_t*)(a.ws + a.wl.snapH) + ((size_t)chain * NI + c) * F * D +
                            (size_t)(col0 + r16) * F + qg * 8;
#pragma unroll
            for (int m = 0; m < FM; ++m) *(bf16x8*)(dst + m * 32) = Ah[m];
        }
        if (jw == 0) {
            float* snapS = (float*)(a.ws + a.wl.snapS) + ((size_t)chain * NI + c) * F;
            int* snapRef = (int*)(a.ws + a.wl.snapRef) + ((size_t)chain * NI + c) * Cp;
            for (int i = tid; i < F; i += NT) snapS[i] = sP[perm_pos(i)];
            for (int i = tid; i < cnt; i += NT) snapRef[i] = cref[i];
            if (tid == 0) ((int*)(a.ws + a.wl.snapN))[(size_t)chain * NI + c] = cnt;
        }

        // ---- candidates: cache slots [0, cnt) then the keys leaving the window ----
        const int64_t eS = ap - w > 0 ? ap - w : 0;
        const int64_t eE = ep - w;
        const int nE = eE > eS ? (int)(eE - eS) : 0;
        const int nU = cnt + nE;
        const int xE0 = (int)(eS - (t0 - w));
        for (int u = tid; u < nU; u += NT) ucode[u] = u < cnt ? cref[u] : xE0 + (u - cnt);
        auto cand_pos = [&](int u) -> int { return u < cnt ? cpos[u] : (int)(eS + (u - cnt)); };
        __syncthreads();  // codes ready

        const bool needSel = nU > C && C > 0;  // the same in every block of the chain
        if (needSel) {
            // ---- partial SRE over this block's 16 columns ----
            const int T = (nU + 15) / 16;
            // Exchange k (k = 1, 2, ...) uses buffer k % 2 and tags every slot with k.
            // A block writes exchange k + 2 only after reading every block's
            // exchange k + 1, which each block writes after reading exchange k, so
            // no slot is overwritten before all blocks have read it.
            const uint32_t tag = arrivals + 1, par = tag & 1u;
            uint64_t* xw = xe + (size_t)(par * KW + jw) * U;
            for (int t0w = wave; t0w < T; t0w += NW * GR) {
                uint4 fh[GR][FM], fl[GR][FM];
                uint2 fv[GR];
#pragma unroll
                for (int k = 0; k < GR; ++k) {
                    int t = t0w + k * NW;
                    t = t < T ? t : T - 1;
                    int u = t * 16 + r16;
                    u = u < nU ? u : nU - 1;
                    const int code = ucode[u];
                    const uint16_t* p = code_phs(code) + qg * 8;
#pragma unroll
                    for (int m = 0; m < FM; ++m) {
                        fh[k][m] = *(const uint4*)(p + m * 32);
                        fl[k][m] = *(const uint4*)(p + F + m * 32);
                    }
                    fv[k] = *(const uint2*)(code_v(code) + col0 + qg * 4);
                }
#pragma unroll
                for (int k = 0; k < GR; ++k) {
                    const int t = t0w + k * NW;
                    if (t >= T) break;  // wave-uniform
                    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f}, acc2 = acc, dac = acc;
#pragma unroll
                    for (int m = 0; m < FM; ++m) {
                        const bf16x8 h = __builtin_bit_cast(bf16x8, fh[k][m]);
                        const bf16x8 l = __builtin_bit_cast(bf16x8, fl[k][m]);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah[m], h, acc, 0, 0, 0);
                        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al[m], h, acc2, 0, 0, 0);
                        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah[m], l, acc2, 0, 0, 0);
                        dac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(As[m], h, dac, 0, 0, 0);
                        dac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(As[m], l, dac, 0, 0, 0);
                    }
                    // rows 0..2 of dac (lane group 0) hold the three parts of d for candidate r16
                    const float dsum = (dac[0] + dac[1]) + dac[2];
                    const float dd = __shfl(dsum, r16, 64);
                    const float inv = dd > 0.f ? 1.0f / dd : 0.f;
                    const float vv[4] = {__uint_as_float(fv[k].x << 16), __uint_as_float(fv[k].x & 0xffff0000u),
                                         __uint_as_float(fv[k].y << 16), __uint_as_float(fv[k].y & 0xffff0000u)};
                    float e = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float df = (acc[i] + acc2[i]) * inv - vv[i];
                        e += df * df;
                    }
                    e += __shfl_xor(e, 16, 64);
                    e += __shfl_xor(e, 32, 64);
                    const int u = t * 16 + r16;
                    if (qg == 0 && u < nU)
                        __hip_atomic_store(&xw[u], ((uint64_t)tag << 32) | __float_as_uint(e), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            }

            // ---- SRE totals: every block's partial for every candidate, added in
            //      column-slice order (the same bits in every block); a slot is
            //      read again until it carries this exchange's tag ----
            ++arrivals;
            {
                const uint64_t* xr = xe + (size_t)par * KW * U;
                uint32_t lo = 0xffffffffu, hi = 0u;
                int ok = 1;
                for (int u = tid; u < nU; u += NT) {
                    uint64_t vals[KW];
#pragma unroll
                    for (int jj = 0; jj < KW; ++jj)
                        vals[jj] = __hip_atomic_load(&xr[(size_t)jj * U + u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    uint32_t polls = 0;
                    for (;;) {
                        bool ready = true;
#pragma unroll
                        for (int jj = 0; jj < KW; ++jj) ready &= (uint32_t)(vals[jj] >> 32) == tag;
                        if (ready) break;
                        if (++polls > kSpinLimit ||
                            __hip_atomic_load(&xsync[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
                            ok = 0;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
#pragma unroll
                        for (int jj = 0; jj < KW; ++jj)
                            if ((uint32_t)(vals[jj] >> 32) != tag)
                                vals[jj] = __hip_atomic_load(&xr[(size_t)jj * U + u], __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT);
                    }
                    if (!ok) break;
                    float e = __uint_as_float((uint32_t)vals[0]);
#pragma unroll
                    for (int jj = 1; jj < KW; ++jj) e += __uint_as_float((uint32_t)vals[jj]);
                    const uint32_t eb = __float_as_uint(e);
                    ebits[u] = eb;
                    lo = min(lo, eb);
                    hi = max(hi, eb);
                }
                lo = wave_min_u32(lo);
                hi = wave_max_u32(hi);
                if (tid == 0) { misc[0] = (int)lo; misc[1] = (int)hi; misc[2] = 0; misc[8] = 1; }
                for (int i = tid; i < NB; i += NT) hist[i] = 0;
                __syncthreads();
                if (!ok) {
                    misc[8] = 0;
                    __hip_atomic_store(&xsync[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(&((StateHeader*)a.state)->fault, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                if (lane == 0 && wave > 0) { atomicMin((uint32_t*)&misc[0], lo); atomicMax((uint32_t*)&misc[1], hi); }
            }
            __syncthreads();
            if (!misc[8]) return;  // block-uniform
            {
                const uint32_t minb = (uint32_t)misc[0];
                const float bscale = (float)NB / ((float)((uint32_t)misc[1] - minb) + 1.0f);
                auto bin_of = [&](uint32_t x) { return min(NB - 1, (int)((float)(x - minb) * bscale)); };
                for (int u = tid; u < nU; u += NT) atomicAdd(&hist[bin_of(ebits[u])], 1);
                __syncthreads();
                int cb[4], tot = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) { cb[k] = hist[NB - 1 - (4 * lane + k)]; tot += cb[k]; }
                int incl = tot;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int up = __shfl_up(incl, o, 64);
                    if (lane >= o) incl += up;
                }
                const int excl = incl - tot;
                int bsel = -1, above = 0;
                if (excl < C && incl >= C) {
                    int cum = excl;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        if (bsel < 0 && cum + cb[k] >= C) { bsel = NB - 1 - (4 * lane + k); above = cum; }
                        cum += cb[k];
                    }
                }
                const uint64_t hit = __ballot(bsel >= 0);
                const int src = __ffsll((long long)hit) - 1;
                const int bstar = __shfl(bsel, src, 64);
                const int need = C - __shfl(above, src, 64);
                for (int u = tid; u < nU; u += NT) {
                    const int bin = bin_of(ebits[u]);
                    if (bin != bstar) keep[u] = bin > bstar;
                    else memb[atomicAdd(&misc[2], 1)] = u;
                }
                __syncthreads();
                const int mm = misc[2];
                for (int i = tid; i < mm; i += NT) {
                    const int u = memb[i];
                    const uint32_t eu = ebits[u];
                    const int pu = cand_pos(u);
                    int rank = 0;
                    for (int j2 = 0; j2 < mm; ++j2) {
                        const int v2 = memb[j2];
                        const uint32_t ev = ebits[v2];
                        rank += (ev > eu) || (ev == eu && cand_pos(v2) < pu);
                    }
                    keep[u] = rank < need;
                }
            }
        } else {
            for (int u = tid; u < nU; u += NT) keep[u] = nU <= C;
        }
        __syncthreads();

        // ---- compaction in candidate order: folded pairs, freed slots, kept leaving keys ----
        {
            const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
            const int nblk = (nU + 63) / 64;
            for (int j = wave; j < nblk; j += NW) {
                const int u = j * 64 + lane;
                const bool valid = u < nU;
                const bool kp = valid && keep[u];
                const int cF = __popcll(__ballot(valid && !kp));
                const int cFr = __popcll(__ballot(valid && u < cnt && !kp));
                const int cK = __popcll(__ballot(valid && u >= cnt && kp));
                if (lane == 0) { bcnt[4 * j] = cF; bcnt[4 * j + 1] = cFr; bcnt[4 * j + 2] = cK; }
            }
            __syncthreads();
            for (int j = wave; j < nblk; j += NW) {
                int oF = 0, oFr = 0, oK = 0;
                for (int j2 = 0; j2 < j; ++j2) { oF += bcnt[4 * j2]; oFr += bcnt[4 * j2 + 1]; oK += bcnt[4 * j2 + 2]; }
                const int u = j * 64 + lane;
                const bool valid = u < nU;
                const bool kp = valid && keep[u];
                const bool isF = valid && !kp;
                const bool isFr = valid && u < cnt && !kp;
                const bool isK = valid && u >= cnt && kp;
                const uint64_t bF = __ballot(isF), bFr = __ballot(isFr), bK = __ballot(isK);
                if (isF) fold[oF + __popcll(bF & lt)] = u;
                if (isFr) freed[oFr + __popcll(bFr & lt)] = u;
                if (isK) keptE[oK + __popcll(bK & lt)] = u;
                if (j == nblk - 1 && lane == 0) {
                    misc[5] = oF + __popcll(bF);
                    misc[6] = oFr + __popcll(bFr);
                    misc[7] = oK + __popcll(bK);
                }
            }
            if (nblk == 0 && tid == 0) { misc[5] = 0; misc[6] = 0; misc[7] = 0; }
        }
        __syncthreads();
        const int nF = misc[5], nFr = misc[6], nK = misc[7];

        // ---- fold into this block's columns: H += phi v^T (phi in three bf16 parts), s += phi ----
        for (int e0 = 0; e0 < nF; e0 += EC) {
            const int ne = nF - e0 < EC ? nF - e0 : EC;
            if (e0 > 0) __syncthreads();  // the previous chunk is consumed
            // two folded rows per thread and feature quad: packed 32-bit LDS writes
            for (int idx = tid; idx < (EC / 2) * (F / 4); idx += NT) {
                const int e2 = (idx % (EC / 2)) * 2, f4 = (idx / (EC / 2)) * 4;
                float x0[4] = {0.f, 0.f, 0.f, 0.f}, x1[4] = {0.f, 0.f, 0.f, 0.f};
                if (e2 < ne) load4(code_phi(ucode[fold[e0 + e2]]) + f4, x0);
                if (e2 + 1 < ne) load4(code_phi(ucode[fold[e0 + e2 + 1]]) + f4, x1);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint16_t a1 = bf16_bits(x0[k]), b1 = bf16_bits(x1[k]);
                    const float ra = x0[k] - bf16_val(a1), rb = x1[k] - bf16_val(b1);
                    const uint16_t a2 = bf16_bits(ra), b2 = bf16_bits(rb);
                    const uint16_t a3 = bf16_bits(ra - bf16_val(a2)), b3 = bf16_bits(rb - bf16_val(b2));
                    uint32_t* row = (uint32_t*)(P + (size_t)(f4 + k) * EP + e2);
                    row[0] = (uint32_t)a1 | ((uint32_t)b1 << 16);
                    row[F * EP / 2] = (uint32_t)a2 | ((uint32_t)b2 << 16);
                    row[F * EP] = (uint32_t)a3 | ((uint32_t)b3 << 16);
                }
            }
            for (int idx = tid; idx < EC * 2; idx += NT) {
                const int e1 = idx >> 1, h8 = (idx & 1) * 8;
                uint4 t4 = make_uint4(0, 0, 0, 0);
                if (e1 < ne) t4 = *(const uint4*)(code_v(ucode[fold[e0 + e1]]) + col0 + h8);
                const uint32_t tw[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
                for (int k = 0; k < 8; ++k) VS[(h8 + k) * EP + e1] = (uint16_t)(tw[k >> 1] >> (16 * (k & 1)));
            }
            __syncthreads();
            if (wave < FT) {
                const bf16x8 ones = __builtin_bit_cast(bf16x8, u16x8{0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80,
                                                                     0x3f80, 0x3f80});
                floatx4 sa = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < EC / 32; ++ks) {
                    const int o = (wave * 16 + r16) * EP + ks * 32 + qg * 8;
                    const bf16x8 p1 = *(const bf16x8*)(P + o);
                    const bf16x8 p2 = *(const bf16x8*)(P + F * EP + o);
                    const bf16x8 p3 = *(const bf16x8*)(P + 2 * F * EP + o);
                    const bf16x8 bv = *(const bf16x8*)(VS + r16 * EP + ks * 32 + qg * 8);
                    Hacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p1, bv, Hacc, 0, 0, 0);
                    Hacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p2, bv, Hacc, 0, 0, 0);
                    Hacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p3, bv, Hacc, 0, 0, 0);
                    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p1, ones, sa, 0, 0, 0);
                    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p2, ones, sa, 0, 0, 0);
                    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p3, ones, sa, 0, 0, 0);
                }
                if (r16 == 0)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sP[perm_pos(wave * 16 + qg * 4 + i)] += sa[i];
            }
        }

        // ---- new operands of H and s; kept leaving keys take freed slots, then new slots ----
        if (nF > 0) {
            if (wave < FT) {
                u16x8 hl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    hl[i] = bf16_bits(Hacc[i]);
                    hl[4 + i] = bf16_bits(Hacc[i] - bf16_val(hl[i]));
                }
                const int pos = perm_pos(wave * 16 + qg * 4);
                *(uint2*)(AX + r16 * AXS + pos) = make_uint2((uint32_t)hl[0] | ((uint32_t)hl[1] << 16),
                                                             (uint32_t)hl[2] | ((uint32_t)hl[3] << 16));
                *(uint2*)(AX + (16 + r16) * AXS + pos) = make_uint2((uint32_t)hl[4] | ((uint32_t)hl[5] << 16),
                                                                    (uint32_t)hl[6] | ((uint32_t)hl[7] << 16));
            }
        }
        for (int i = tid; i < nK; i += NT) {
            const int u = keptE[i];
            const int slot = i < nFr ? freed[i] : cnt + (i - nFr);
            cref[slot] = xE0 + (u - cnt);
            cpos[slot] = (int)(eS + (u - cnt));
        }
        cnt = nU < C ? nU : C;
        __syncthreads();
        if (nF > 0) {
#pragma unroll
            for (int m = 0; m < FM; ++m) {
                Ah[m] = *(const bf16x8*)(AX + r16 * AXS + m * 32 + qg * 8);
                Al[m] = *(const bf16x8*)(AX + (16 + r16) * AXS + m * 32 + qg * 8);
            }
            build_As();
        }
    }

    // ---- state out: this block's rows of H^T; block 0 also s, cache and window ----
    if (wave < FT)
        *(float4*)(ch.H() + (size_t)(col0 + r16) * F + wave * 16 + qg * 4) =
            make_float4(Hacc[0], Hacc[1], Hacc[2], Hacc[3]);
    if (jw != 0) return;
    if (tid == 0) {
        uint32_t polls = 0;
        while (__hip_atomic_load(&xsync[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)KW) {
            if (__hip_atomic_load(&xsync[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u || ++polls > kSpinLimit) {
                __hip_atomic_store(&xsync[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&((StateHeader*)a.state)->fault, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
    for (int i = tid; i < F; i += NT) ch.s()[i] = sP[perm_pos(i)];
    for (int i = tid; i < cnt; i += NT) ch.cpos()[i] = cpos[i];
    for (int idx = tid; idx < cnt * D; idx += NT) {
        const int i = idx / D, j = idx % D;
        if (cref[i] >= 0) {
            ch.cache_k<bf16>()[(size_t)i * D + j] = xrow_k<bf16>(a, chain, b, g, cref[i])[j];
            ch.cache_v<bf16>()[(size_t)i * D + j] = xrow_v<bf16>(a, chain, b, g, cref[i])[j];
        }
    }
    if (w > 0) {
        const int64_t tend = t0 + n;
        const int64_t p0 = tend - w > t0 ? tend - w : t0;
        const int nr = (int)(tend - p0);
        for (int idx = tid; idx < nr * D; idx += NT) {
            const int i = idx / D, j = idx % D;
            const int64_t p = p0 + i;
            const int slot = (int)(p % w);
            const size_t src = (((size_t)b * n + (size_t)(p - t0)) * d.Hkv + g) * D + j;
            ch.ring_k<bf16>()[(size_t)slot * D + j] = ((const bf16*)a.k)[src];
            ch.ring_v<bf16>()[(size_t)slot * D + j] = ((const bf16*)a.v)[src];
        }
    }
    if (tid == 0) {
        ch.cnt() = cnt;
        ch.tok() = t0 + n;
    }
}

}  // namespace lola
