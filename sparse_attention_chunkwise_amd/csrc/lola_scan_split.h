// Interval scan with each (sequence, KV head) chain spread over D/16 x PU
// workgroups (bf16 io): D/16 column slices of H times PU = 4, 2 or 1
// candidate groups, as many as the device holds at once.
//
// The scan of one chain is a recurrence over update intervals: the SRE of the
// cached and leaving pairs is scored against the interval-start state, the
// highest C stay, the rest are folded (LoLA technical summary, gist.science,
// sections "Het Self-Recall Error (SRE) Mechanisme" and "Inferentiestrategie").
// With few chains (one sequence, 8 KV heads) one workgroup per chain leaves
// most of the chip idle and puts every step of an interval on one CU.  Here
// workgroup (j, u) of a chain owns columns [16j, 16j + 16) of H and the
// candidate tiles u, u + PU, ...:
//
//   * its 4 waves split those tiles (16 candidates, one MFMA tile each); a
//     wave computes n = H^T phi(k) for its 16 columns with bf16 MFMAs on hi/lo
//     parts (hi.hi + lo.hi + hi.lo) and d = s . phi(k) with an MFMA whose A
//     rows are the three bf16 parts of s (d is s in fp32 times phi hi + lo),
//     and publishes the partial error sum_{its columns} (n/d - v)^2;
//   * partials travel through the workspace as 64-bit slots (exchange number,
//     value) written and polled with agent-scope relaxed atomics, so no fence
//     or cache flush is needed; every workgroup adds the D/16 partials in the
//     same order and takes the same keep / fold decision;
//   * wave 0 selects with a bracketing threshold search over the SRE bit
//     patterns held in registers (started from the previous interval's
//     threshold, steps interpolated from the ballot counts, no LDS round
//     trips), then compacts;
//   * each workgroup folds the chosen pairs into its own columns only (phi hi +
//     lo, 16 significant bits) and keeps s, which every workgroup updates
//     identically.  Barriers inside the interval order LDS only, so global
//     loads stay in flight across them.
//
// Block b runs on XCD b % 8 (round-robin dispatch), so the workgroups of a
// chain are placed on one XCD and meet in its L2.  The launch is
// cooperative, so all of them are resident together; a wait that does not end
// within a fixed number of polls marks the state as faulted and returns.
#pragma once

#include <climits>
#include <type_traits>

#include "lola_prefill.h"

namespace lola {

constexpr int kSplitThreads = 256;                    // 4 waves, one per SIMD
constexpr int kSplitGroup = 5;                        // candidate tiles per wave per load round
constexpr uint32_t kSpinLimit = 1u << 22;

struct SplitSmem {
    size_t PR, VS, AX, s, sparts, ebits, foldc, cref, cpos, freed, tiep, misc, total;
};

// Every array is sized for the largest cache and chunk, so that all offsets are
// compile-time constants (immediate LDS offsets, no base registers).
template <int F>
__host__ __device__ constexpr SplitSmem split_smem()
{
    SplitSmem m{};
    constexpr int EP = kFoldChunk + 8;
    size_t off = 0;
    m.PR = off;     off += align_up(sizeof(uint16_t) * 2 * (size_t)F * EP, 16);        // [2F][EP]
    m.VS = off;     off += align_up(sizeof(uint16_t) * 16 * (size_t)EP, 16);          // [16][EP]
    m.AX = off;     off += align_up(sizeof(uint16_t) * 2 * 16 * (size_t)(F + 8), 16); // [2][16][F+8]
    m.s = off;      off += align_up(sizeof(float) * F, 16);
    m.sparts = off; off += align_up(sizeof(uint16_t) * 3 * (size_t)F, 16);            // [3][F]
    m.ebits = off;  off += sizeof(uint32_t) * kMaxCand;
    m.foldc = off;  off += sizeof(int) * kMaxCand;
    m.cref = off;   off += sizeof(int) * kMaxCache;
    m.cpos = off;   off += sizeof(int) * kMaxCache;
    m.freed = off;  off += sizeof(int) * kMaxCache;
    m.tiep = off;   off += sizeof(int) * kMaxCand;
    m.misc = off;   off += sizeof(int) * 16;
    m.total = align_up(off, 16);
    return m;
}

// Grid of the split scan: 8 * (D/16) * PU * ceil(chains / 8) blocks, PU candidate
// groups per column slice.
__host__ __device__ inline int split_blocks(int D, int chains, int PU) { return 8 * (D / 16) * PU * ((chains + 7) / 8); }

template <int D, int F>
__global__ __launch_bounds__(kSplitThreads) void scan_split_kernel(Args a)
{
    constexpr int KW = D / 16, NT = kSplitThreads, NW = NT / 64, FT = F / 16, FM = F / 32;
    constexpr int EC = kFoldChunk, EP = EC + 8, AXS = F + 8, GR = kSplitGroup;
    constexpr int RES = NW * GR, HT = (FT + NW - 1) / NW;
    static_assert(EC * 4 == NT && EC == 64 && (2 * F / 8) % (2 * NW) == 0, "fold staging covers the chunk exactly");
    static_assert(5 * 64 <= kMaxCache && 5 * 64 <= kMaxCand, "register selection reads 5 chunks of cref and ebits");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    // header fields other than `fault` are the same for every block of the launch, so
    // a mismatch returns every block at once; `fault` is tested below, block-uniformly
    if (!state_ok(a, true)) return;
    const Dims& d = a.d;
    const int w = d.w, C = d.C, L = d.L;
    const int chains = a.B * d.Hkv;
    const int PU = (int)gridDim.x / (8 * KW * ((chains + 7) / 8));  // candidate groups: 1, 2 or 4
    const int pl = __builtin_ctz((unsigned)PU);                      // log2 PU (shifts, not divisions)
    const int bid = blockIdx.x, xcd = bid & 7, sb = bid >> 3;
    const int jw = sb % KW, ju = (sb / KW) & (PU - 1), chain = ((sb / KW) >> pl) * 8 + xcd;
    const bool lead = ju == 0;  // writes this column slice's rows of the snapshots and of H
    if (chain >= chains) return;  // the whole chain is absent: none of its blocks waits
    const int col0 = 16 * jw;
    constexpr SplitSmem sm = split_smem<F>();
    uint16_t* PR = (uint16_t*)(smem + sm.PR);      // folded pairs transposed: row = phi hi | lo slot, column = pair
    uint16_t* VS = (uint16_t*)(smem + sm.VS);      // folded pairs' values, this block's 16 columns, transposed
    uint16_t* AX = (uint16_t*)(smem + sm.AX);      // hi, lo of H^T rows col0.. (operand order)
    float* sP = (float*)(smem + sm.s);             // s, operand order
    uint16_t* sParts = (uint16_t*)(smem + sm.sparts);
    uint32_t* ebits = (uint32_t*)(smem + sm.ebits);
    int* foldc = (int*)(smem + sm.foldc);          // fold index -> candidate code
    int* cref = (int*)(smem + sm.cref);
    int* cpos = (int*)(smem + sm.cpos);
    int* freed = (int*)(smem + sm.freed);
    int* tiep = (int*)(smem + sm.tiep);
    int* misc = (int*)(smem + sm.misc);

    const int b = chain / d.Hkv, g = chain % d.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, qg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps wave branches scalar
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    Chain ch = chain_of(a, chain);
    const int64_t t0 = ws_t0(a, b);
    const int n = a.n, NI = a.NI;  // rows per sequence in k, v; snapshot slots per chain
    const int ns = seq_tokens(a, b), NIs = (ns + L - 1) / L;  // this sequence's tokens and intervals
    const int Cp = C > 0 ? C : 1;
    const int U = C + L;
    uint32_t* xsync = (uint32_t*)(a.ws + a.wl.xsync) + (size_t)chain * 16;
    uint64_t* xe = (uint64_t*)(a.ws + a.wl.xe) + (size_t)chain * 2 * KW * U;

    // ---- state in ----
    const float* Hst = ch.H();  // H^T [D][F]
    // Hacc[h][i] = H[ft*16 + qg*4 + i][col0 + r16] for the wave's feature tiles ft = wave + NW*h
    floatx4 Hacc[HT];
#pragma unroll
    for (int h = 0; h < HT; ++h) Hacc[h] = floatx4{0.f, 0.f, 0.f, 0.f};
    {
        float hv[FT][4];
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) load4(Hst + (size_t)(col0 + r16) * F + ft * 16 + qg * 4, hv[ft]);
#pragma unroll
        for (int ft = 0; ft < FT; ++ft)
            if (ft % NW == wave) Hacc[ft / NW] = floatx4{hv[ft][0], hv[ft][1], hv[ft][2], hv[ft][3]};
        if (wave == 0) {
#pragma unroll
            for (int m = 0; m < FM; ++m) {
                u16x8 h, l;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float x = hv[2 * m + (j >> 2)][j & 3];
                    h[j] = bf16_bits(x);
                    l[j] = bf16_bits(x - bf16_val(h[j]));
                }
                *(u16x8*)(AX + r16 * AXS + m * 32 + qg * 8) = h;
                *(u16x8*)(AX + (16 + r16) * AXS + m * 32 + qg * 8) = l;
            }
        }
    }
    auto split3 = [&](int pos) {  // the three bf16 parts of s at operand position pos
        const float x = sP[pos];
        const uint16_t p1 = bf16_bits(x);
        const float r1 = x - bf16_val(p1);
        const uint16_t p2 = bf16_bits(r1);
        sParts[pos] = p1;
        sParts[F + pos] = p2;
        sParts[2 * F + pos] = bf16_bits(r1 - bf16_val(p2));
    };
    // A operands of the SRE from LDS: H^T hi and lo rows of this block's columns,
    // and for d rows 4q, 4q+1, 4q+2 = the three bf16 parts of s (q = 0..3), the
    // others zero, so that every lane group receives d in its own result rows
    auto load_A = [&](bf16x8* Ah, bf16x8* Al, bf16x8* As) {
        const int row = (r16 & 3) < 3 ? (r16 & 3) : 2;
        const uint32_t keepm = (r16 & 3) < 3 ? 0xffffffffu : 0u;
#pragma unroll
        for (int m = 0; m < FM; ++m) {
            Ah[m] = *(const bf16x8*)(AX + r16 * AXS + m * 32 + qg * 8);
            Al[m] = *(const bf16x8*)(AX + (16 + r16) * AXS + m * 32 + qg * 8);
            uint4 x = *(const uint4*)(sParts + row * F + m * 32 + qg * 8);
            x.x &= keepm;
            x.y &= keepm;
            x.z &= keepm;
            x.w &= keepm;
            As[m] = __builtin_bit_cast(bf16x8, x);
        }
    };
    for (int i = tid; i < F; i += NT) sP[perm_pos(i)] = ch.s()[i];
    int cnt = min(max(ch.cnt(), 0), C);
    for (int i = tid; i < cnt; i += NT) {
        cpos[i] = ch.cpos()[i];
        cref[i] = -(i + 1);
    }
    if (tid == 0) {
        misc[8] = 0;
        misc[9] = __hip_atomic_load(&((StateHeader*)a.state)->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // (a full barrier: it also waits until every wave's loads of H, s, the count and
    // the positions have returned, before the count below says they are read)
    __syncthreads();
    // An earlier call left the state faulted: write nothing.  Every block sees that
    // fault word (an earlier launch wrote it), so none of them waits for another; a
    // block that sees it set by a sibling of this launch (one that gave up waiting)
    // finds the give-up flag xsync[1] already raised for the others.
    if (misc[9] != 0) return;
    for (int i = tid; i < F; i += NT) split3(i);
    // the lead blocks rewrite H, and block 0 also s, the count and the cache positions,
    // at the end: they wait until every block of the chain has read them (counter xsync[2])
    if (tid == 0) __hip_atomic_fetch_add(&xsync[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    const uint16_t* phiS0 = ws_phiS(a, chain, 0);
    const uint16_t* cphiS0 = ws_cphiS(a, chain, 0);
    const bf16* vin0 = (const bf16*)a.v + ((size_t)b * n * d.Hkv + g) * D;
    const bf16* ring0v = (const bf16*)(a.ws + a.wl.ring0_v) + (size_t)chain * w * D;
    const bf16* cache0v = (const bf16*)(a.ws + a.wl.cache0_v) + (size_t)chain * Cp * D;
    auto code_phs = [&](int code) -> const uint16_t* {
        return code >= 0 ? phiS0 + (size_t)code * 2 * F : cphiS0 + (size_t)(-code - 1) * 2 * F;
    };
    auto code_v = [&](int code) -> const bf16* {
        const bf16* pin = vin0 + (size_t)(code - w) * d.Hkv * D;
        const bf16* pring = ring0v + (size_t)code * D;
        const bf16* pcache = cache0v + (size_t)(-code - 1) * D;
        return code >= w ? pin : (code >= 0 ? pring : pcache);
    };
    // interval c is [ap, ep); its leaving keys [eS, eS + nE) are X rows xE0 ..
    struct Iv {
        int64_t eS;
        int nE, xE0;
    };
    auto interval = [&](int c) -> Iv {
        const int64_t ap = t0 + (int64_t)c * L;
        const int64_t ep = ap + L < t0 + ns ? ap + L : t0 + ns;
        Iv v;
        v.eS = ap - w > 0 ? ap - w : 0;
        const int64_t eE = ep - w;
        v.nE = eE > v.eS ? (int)(eE - v.eS) : 0;
        v.xE0 = (int)(v.eS - (t0 - w));
        return v;
    };

    // Candidate u of an interval whose cache holds cntq pairs and whose leaving keys
    // start at extended row xq: the pair in slot u (u < cntq), else leaving key u - cntq.
    // Codes: >= 0 an extended row of this call, < 0 slot -code - 1 of the call-start cache.
    auto cand_code = [&](int u, int cntq, int xq) -> int { return u < cntq ? cref[u] : xq + (u - cntq); };

    // Tiles of the prefetched path (at most 2 NW - 1 per block): block tile i = wave
    // in slot 0, and i = NW + wave - 1 in slot 1 for waves 1.. (wave 0 runs the
    // selection and keeps one tile); -1 = no tile
    auto two_tile = [&](int k) -> int { return k == 0 ? wave : (wave > 0 ? NW + wave - 1 : -1); };

    // Partial SRE of this block's candidate tiles t = ju + PU * i, i = ibase + wave +
    // NW * k (k < G): sre_load fetches the phi rows (hi, lo) and the values of a
    // wave's G tiles, sre_math computes them two at a time and publishes the
    // partial errors.
    auto sre_load = [&](auto gTag, int cntq, int xq, int nUq, int ibase, uint4 (&fh)[decltype(gTag)::value][FM],
                        uint4 (&fl)[decltype(gTag)::value][FM], uint2 (&fv)[decltype(gTag)::value]) {
        constexpr int G = decltype(gTag)::value;
        const int T = (nUq + 15) / 16;
#pragma unroll
        for (int k = 0; k < G; ++k) {
            int t = ju + PU * (ibase + wave + k * NW);
            t = t < T ? t : T - 1;
            int u = t * 16 + r16;
            u = u < nUq ? u : nUq - 1;
            const int code = cand_code(u, cntq, xq);
            const uint16_t* p = code_phs(code) + qg * 8;
#pragma unroll
            for (int m = 0; m < FM; ++m) {
                fh[k][m] = *(const uint4*)(p + m * 32);
                fl[k][m] = *(const uint4*)(p + F + m * 32);
            }
            fv[k] = *(const uint2*)(code_v(code) + col0 + qg * 4);
        }
    };
    auto sre_math = [&](auto gTag, int nUq, int ibase, uint64_t* xw, uint32_t tag, const bf16x8* Ah,
                        const bf16x8* Al, const bf16x8* As, const uint4 (&fh)[decltype(gTag)::value][FM],
                        const uint4 (&fl)[decltype(gTag)::value][FM], const uint2 (&fv)[decltype(gTag)::value]) {
        constexpr int G = decltype(gTag)::value;
        const int T = (nUq + 15) / 16;
        // two tiles at a time, m outer: consecutive MFMAs are independent
#pragma unroll
        for (int k0 = 0; k0 < G; k0 += 2) {
            constexpr int P = 2;
            floatx4 acc[P], acc2[P], dac[P];
#pragma unroll
            for (int q = 0; q < P; ++q) acc[q] = acc2[q] = dac[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < FM; ++m)
#pragma unroll
                for (int q = 0; q < P; ++q) {
                    const int k = k0 + q < G ? k0 + q : G - 1;
                    const bf16x8 h = __builtin_bit_cast(bf16x8, fh[k][m]);
                    const bf16x8 l = __builtin_bit_cast(bf16x8, fl[k][m]);
                    acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah[m], h, acc[q], 0, 0, 0);
                    acc2[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al[m], h, acc2[q], 0, 0, 0);
                    dac[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(As[m], h, dac[q], 0, 0, 0);
                    acc2[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah[m], l, acc2[q], 0, 0, 0);
                    dac[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(As[m], l, dac[q], 0, 0, 0);
                }
#pragma unroll
            for (int q = 0; q < P; ++q) {
                const int k = k0 + q < G ? k0 + q : G - 1;
                const int it = G == 2 ? two_tile(k0 + q) : ibase + wave + (k0 + q) * NW;
                const int t = it >= 0 ? ju + PU * it : T;
                // rows 4qg .. 4qg+2 of dac hold the three parts of d for candidate r16
                const float dd = (dac[q][0] + dac[q][1]) + dac[q][2];
                const float inv = dd > 0.f ? __builtin_amdgcn_rcpf(dd) : 0.f;
                const float vv[4] = {__uint_as_float(fv[k].x << 16), __uint_as_float(fv[k].x & 0xffff0000u),
                                     __uint_as_float(fv[k].y << 16), __uint_as_float(fv[k].y & 0xffff0000u)};
                float e = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float df = (acc[q][i] + acc2[q][i]) * inv - vv[i];
                    e += df * df;
                }
                e = quad_sum(e);
                const int u = t * 16 + r16;
                if (qg == 0 && k0 + q < G && t < T && u < nUq)
                    __hip_atomic_store(&xw[u], ((uint64_t)tag << 32) | __float_as_uint(e), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    };

    uint32_t arrivals = 0;  // exchanges this block has completed
    uint32_t tauPrev = 0u;  // threshold of the previous selection (wave 0)
    // Operands of the next SRE when each wave has at most two tiles, loaded while
    // the previous interval folds.  A lane keeps the candidate code of the row it
    // holds per tile (pfcode): cache slots mostly keep their pair from one interval
    // to the next and a tile always maps to the same wave, so only rows whose code
    // changed are loaded again.  Where the next SRE is not needed or loads its own
    // operands, and in a wave's tile slot past the last tile (its results are not
    // stored), the row of candidate code 0 (extended row 0, always present) is held.
    using Two = std::integral_constant<int, 2>;
    uint4 pfh[2][FM], pfl[2][FM];
    uint2 pfv[2];
    int pfcode[2] = {INT_MIN, INT_MIN};
    auto tiles_of_block = [&](int nUq) { const int T = (nUq + 15) / 16; return T > ju ? (T - ju + PU - 1) >> pl : 0; };
    auto prefetch_next = [&](int nUq, int cntq, int xq) {
        const bool use = nUq > C && C > 0 && tiles_of_block(nUq) <= 2 * NW - 1;
        const int T = (nUq + 15) / 16;
        int code[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {  // a tile slot past the last tile holds the code-0 row
            const int it = two_tile(k), t = it >= 0 ? ju + PU * it : T;
            int u = t * 16 + r16;
            u = u < nUq ? u : nUq - 1;
            code[k] = use && t < T ? cand_code(u, cntq, xq) : 0;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k)
            if (code[k] != pfcode[k]) {
                const uint16_t* p = code_phs(code[k]) + qg * 8;
#pragma unroll
                for (int m = 0; m < FM; ++m) {
                    pfh[k][m] = *(const uint4*)(p + m * 32);
                    pfl[k][m] = *(const uint4*)(p + F + m * 32);
                }
                pfv[k] = *(const uint2*)(code_v(code[k]) + col0 + qg * 4);
                pfcode[k] = code[k];
            }
    };
    // the same for the rows of leaving keys only, whose codes are known before the
    // selection (waves 1.. load them while wave 0 selects)
    auto prefetch_new = [&](int nUq, int cntq, int xq) {
        const bool use = nUq > C && C > 0 && tiles_of_block(nUq) <= 2 * NW - 1;
        const int T = (nUq + 15) / 16;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int it = two_tile(k), t = it >= 0 ? ju + PU * it : T;
            int u = t * 16 + r16;
            u = u < nUq ? u : nUq - 1;
            const int code = xq + (u - cntq);
            if (use && t < T && u >= cntq && code != pfcode[k]) {
                const uint16_t* p = code_phs(code) + qg * 8;
#pragma unroll
                for (int m = 0; m < FM; ++m) {
                    pfh[k][m] = *(const uint4*)(p + m * 32);
                    pfl[k][m] = *(const uint4*)(p + F + m * 32);
                }
                pfv[k] = *(const uint2*)(code_v(code) + col0 + qg * 4);
                pfcode[k] = code;
            }
        }
    };
    {
        const Iv v0 = interval(0);
        prefetch_next(cnt + v0.nE, cnt, v0.xE0);
    }

    for (int c = 0; c < NIs; ++c) {
        const Iv iv = interval(c);
        const int64_t eS = iv.eS;
        const int nE = iv.nE, xE0 = iv.xE0;
        const int nU = cnt + nE;
        const int T = (nU + 15) / 16;

        // ---- interval-start snapshot: H^T hi parts of this block's rows, s and cache
        //      refs (written before the fold and the slot update change them) ----
        // (the blocks of a column slice hold identical rows, and every block the
        // same s and slot codes, so the writes are spread: block ju writes the
        // 32-feature pieces m with m % PU == ju, two other blocks s and the refs).
        // Threads t0 .. NT - 1 write it: waves 1.. while wave 0 selects, or all.
        auto snapshot = [&](int t0) {
            if (wave == 1) {
                uint16_t* dst = (uint16_t*)(a.ws + a.wl.snapH) + ((size_t)chain * NI + c) * F * D +
                                (size_t)(col0 + r16) * F + qg * 8;
#pragma unroll
                for (int m = 0; m < FM; ++m)
                    if ((m & (PU - 1)) == ju) *(uint4*)(dst + m * 32) = *(const uint4*)(AX + r16 * AXS + m * 32 + qg * 8);
            }
            if (jw == 1 % KW && ju == (1 & (PU - 1))) {
                float* snapS = (float*)(a.ws + a.wl.snapS) + ((size_t)chain * NI + c) * F;
                for (int i = tid - t0; i < F; i += NT - t0) snapS[i] = sP[perm_pos(i)];
            }
            if (jw == 2 % KW && ju == (2 & (PU - 1))) {
                int* snapRef = (int*)(a.ws + a.wl.snapRef) + ((size_t)chain * NI + c) * Cp;
                for (int i = tid - t0; i < cnt; i += NT - t0) snapRef[i] = cref[i];
                if (tid == t0) ((int*)(a.ws + a.wl.snapN))[(size_t)chain * NI + c] = cnt;
            }
        };

        const bool needSel = nU > C && C > 0;  // the same in every block of the chain
        if (needSel) {
            // ---- partial SRE over this block's 16 columns ----
            // Exchange k (k = 1, 2, ...) uses buffer k % 2 and tags every slot with k.
            // A block writes exchange k + 2 only after reading every block's
            // exchange k + 1, which each block writes after reading exchange k, so
            // no slot is overwritten before all blocks have read it.
            const uint32_t tag = arrivals + 1, par = tag & 1u;
            uint64_t* xw = xe + (size_t)(par * KW + jw) * U;
            {
                bf16x8 Ah[FM], Al[FM], As[FM];
                load_A(Ah, Al, As);
                const int TB = tiles_of_block(nU);
                if (TB <= 2 * NW - 1)  // operands loaded during the previous fold (or before the loop)
                    sre_math(Two{}, nU, 0, xw, tag, Ah, Al, As, pfh, pfl, pfv);
                else
                    for (int ib = 0; ib < TB; ib += RES) {
                        uint4 fh[GR][FM], fl[GR][FM];
                        uint2 fv[GR];
                        sre_load(std::integral_constant<int, GR>{}, cnt, xE0, nU, ib, fh, fl, fv);
                        sre_math(std::integral_constant<int, GR>{}, nU, ib, xw, tag, Ah, Al, As, fh, fl, fv);
                    }
            }
            ++arrivals;

            // ---- SRE totals: every block's partial, added in column-slice order
            //      (the same bits in every block); a slot is read again until it
            //      carries this exchange's tag ----
            const uint64_t* xr = xe + (size_t)par * KW * U;
            int ok = 1;
            for (int u0 = tid; u0 < nU; u0 += 2 * NT) {
                // two candidates per pass, so that their loads are in flight together
                const int u1 = u0 + NT < nU ? u0 + NT : u0;
                uint64_t va[KW], vb[KW];
#pragma unroll
                for (int jj = 0; jj < KW; ++jj) {
                    va[jj] = __hip_atomic_load(&xr[(size_t)jj * U + u0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    vb[jj] = __hip_atomic_load(&xr[(size_t)jj * U + u1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                uint32_t polls = 0;
                for (;;) {
                    bool ready = true;
#pragma unroll
                    for (int jj = 0; jj < KW; ++jj)
                        ready &= (uint32_t)(va[jj] >> 32) == tag && (uint32_t)(vb[jj] >> 32) == tag;
                    if (ready) break;
                    // the give-up flag costs a round trip of its own: it is read every
                    // 64th pass only
                    if ((++polls & 63u) == 0u &&
                        (polls > kSpinLimit ||
                         __hip_atomic_load(&xsync[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)) {
                        ok = 0;
                        break;
                    }
                    // read every slot again (a ready slot keeps its value until exchange k + 2)
#pragma unroll
                    for (int jj = 0; jj < KW; ++jj) {
                        va[jj] = __hip_atomic_load(&xr[(size_t)jj * U + u0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        vb[jj] = __hip_atomic_load(&xr[(size_t)jj * U + u1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
                if (!ok) break;
                float e0 = __uint_as_float((uint32_t)va[0]), e1 = __uint_as_float((uint32_t)vb[0]);
#pragma unroll
                for (int jj = 1; jj < KW; ++jj) {
                    e0 += __uint_as_float((uint32_t)va[jj]);
                    e1 += __uint_as_float((uint32_t)vb[jj]);
                }
                ebits[u0] = __float_as_uint(e0);
                ebits[u1] = __float_as_uint(e1);
            }
            if (!ok) {
                misc[8] = (int)tag;  // this exchange failed
                __hip_atomic_store(&xsync[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&((StateHeader*)a.state)->fault, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            lds_sync();
            if (misc[8] == (int)tag) return;  // block-uniform
        } else
            snapshot(0);

        // ---- wave 0: exact top-C on (SRE desc, position asc), compaction, slot
        //      updates and the next interval's candidate list ----
        const int cntN = nU < C ? nU : C;
        const Iv ivN = interval(c + 1 < NIs ? c + 1 : c);
        const int nUN = c + 1 < NIs ? cntN + ivN.nE : 0;
        uint32_t kbits = 0u;  // wave 0: bit i set = the lane's candidate of chunk i stays
        // Slot update (wave 0, while the fold rows load): folded cache pairs free their
        // slots in slot order, and the kept leaving keys take the freed slots in order,
        // then new slots past the count.
        auto slot_update = [&]() {
            int nFr = 0;
            for (int i = 0; i < (cnt + 63) / 64; ++i) {
                const int u = i * 64 + lane;
                const bool isFr = u < cnt && !((kbits >> i) & 1u);
                const uint64_t b = __ballot(isFr);
                if (isFr) freed[nFr + __popcll(b & lt)] = u;
                nFr += __popcll(b);
            }
            lds_wait();
            int nK = 0;
            for (int i = cnt / 64; i < (nU + 63) / 64; ++i) {
                const int u = i * 64 + lane;
                const bool isK = u >= cnt && u < nU && ((kbits >> i) & 1u);
                const uint64_t bK = __ballot(isK);
                if (isK) {
                    const int ki = nK + __popcll(bK & lt);
                    const int slot = ki < nFr ? freed[ki] : cnt + (ki - nFr);
                    cref[slot] = xE0 + (u - cnt);
                    cpos[slot] = (int)(eS + (u - cnt));
                }
                nK += __popcll(bK);
            }
        };
        if (wave == 0) {
            auto cand_pos = [&](int u) -> int { return u < cnt ? cpos[u] : (int)(eS + (u - cnt)); };
            // NC = candidate chunks of 64 held per lane (a compile-time bound >= ceil(nU / 64))
            auto select_compact = [&](auto ncTag) {
                constexpr int NC = decltype(ncTag)::value;
                uint32_t key[NC];
                int ucv[NC];              // candidate codes
                uint64_t km[NC], vm[NC];  // keep and valid masks per chunk
                // (both arrays hold at least 64 NC entries: the loads need no branch)
                uint32_t eb[NC];
                int cr[NC];
#pragma unroll
                for (int i = 0; i < NC; ++i) {
                    eb[i] = ebits[i * 64 + lane];
                    cr[i] = cref[i * 64 + lane];
                }
                // (all ten reads issued before the first wait)
#pragma unroll
                for (int i = 0; i < NC; ++i) asm volatile("" : "+v"(eb[i]), "+v"(cr[i]));
#pragma unroll
                for (int i = 0; i < NC; ++i) {
                    const int u = i * 64 + lane;
                    key[i] = u < nU ? eb[i] : 0u;
                    ucv[i] = u < cnt ? cr[i] : xE0 + (u - cnt);
                    vm[i] = __ballot(u < nU);
                    km[i] = (!needSel && nU <= C) ? vm[i] : 0ull;
                }
                if (needSel) {
                    // Threshold: the largest t with #{key >= t} >= C (keys are SRE bit
                    // patterns, order-preserving since SRE >= 0; slots past nU hold 0).
                    // The bracket lo < hi keeps count(lo) >= C > count(hi).  It starts
                    // from the previous interval's threshold, widens by steps that grow
                    // 4x until it encloses the new one, then narrows at the point where
                    // the count is expected to cross C (linear in the bit pattern), with
                    // a halving step whenever two steps did not halve the bracket.  It
                    // stops once exactly C keys reach lo, or when hi = lo + 1 (then lo
                    // is the C-th largest key).  lo, hi and the counts are wave-uniform.
                    uint32_t lo = 0u, hi = 0x80000000u;  // no non-negative pattern reaches hi
                    int clo = nU, chi = 0;
                    auto probe = [&](uint32_t t) -> int {
                        uint64_t bal[NC];  // all compares first, then the counts
#pragma unroll
                        for (int i = 0; i < NC; ++i) bal[i] = __ballot(key[i] >= t);
                        int cc = 0;
#pragma unroll
                        for (int i = 0; i < NC; ++i) cc += __popcll(bal[i]);
                        cc = __builtin_amdgcn_readfirstlane(cc);
                        if (cc >= C) {
                            lo = t;
                            clo = cc;
                        } else {
                            hi = t;
                            chi = cc;
                        }
                        return cc;
                    };
                    int cc = probe(tauPrev > 0u && tauPrev < hi ? tauPrev : 0x3f800000u);
                    uint32_t step = 1u << 18;
#pragma nounroll
                    while (cc != C && hi - lo > 2u * step) {
                        cc = probe(cc >= C ? lo + step : hi - step);
                        step = step < (1u << 28) ? step << 2 : step;
                    }
                    uint32_t wprev = 0xffffffffu;
                    int k = 0;
#pragma nounroll
                    while (cc != C && hi - lo > 1u) {
                        const uint32_t wd = hi - lo;
                        uint32_t t;
                        if ((k & 1) && wd > wprev / 2u)
                            t = lo + wd / 2u;
                        else {
                            const float frac = ((float)(clo - C) + 0.5f) * __builtin_amdgcn_rcpf((float)(clo - chi));
                            t = lo + (uint32_t)((float)wd * frac);
                            t = t <= lo ? lo + 1u : (t >= hi ? hi - 1u : t);
                            t = __builtin_amdgcn_readfirstlane(t);
                        }
                        if (!(k & 1)) wprev = wd;
                        ++k;
                        cc = probe(t);
                    }
                    uint32_t tau = lo;
                    const int ge = clo;
                    tauPrev = lo;
                    const bool exact = ge == C;
                    int above = 0, ties = 0;
                    if (!exact) {
#pragma unroll
                        for (int i = 0; i < NC; ++i) {
                            above += __popcll(__ballot(key[i] > tau) & vm[i]);
                            ties += __popcll(__ballot(key[i] == tau) & vm[i]);
                        }
                    }
                    const int need = C - above;
#pragma unroll
                    for (int i = 0; i < NC; ++i) km[i] = __ballot(key[i] >= tau) & vm[i];
                    if (!exact && ties > need) {
                        // equal SRE at the boundary: the older positions stay
                        int nt = 0;
#pragma unroll
                        for (int i = 0; i < NC; ++i) {
                            const bool tie = ((vm[i] >> lane) & 1ull) && key[i] == tau;
                            const uint64_t bm = __ballot(tie);
                            if (tie) tiep[nt + __popcll(bm & lt)] = cand_pos(i * 64 + lane);
                            nt += __popcll(bm);
                        }
                        lds_wait();
#pragma unroll
                        for (int i = 0; i < NC; ++i) {
                            const int u = i * 64 + lane;
                            const bool tie = ((vm[i] >> lane) & 1ull) && key[i] == tau;
                            int rank = 0;
                            if (tie) {
                                const int p = cand_pos(u);
                                for (int j = 0; j < nt; ++j) rank += tiep[j] < p;
                            }
                            km[i] = __ballot(key[i] > tau || (tie && rank < need)) & vm[i];
                        }
                    }
                }
                // fold list in candidate order; the keep bits go to the slot update
                int nF = 0;
#pragma unroll
                for (int i = 0; i < NC; ++i) {
                    const bool isF = ((vm[i] & ~km[i]) >> lane) & 1ull;
                    const uint64_t bF = __ballot(isF);
                    if (isF) foldc[nF + __popcll(bF & lt)] = ucv[i];
                    nF += __popcll(bF);
                }
                uint32_t kb = 0u;
#pragma unroll
                for (int i = 0; i < NC; ++i) kb |= (uint32_t)((km[i] >> lane) & 1ull) << i;
                kbits = kb;
                if (lane == 0) misc[5] = nF;
            };
            // The same selection for more than 5 chunks, with runtime loops over the
            // chunks and the keys read from LDS at each use: no per-chunk registers, so
            // the wide case does not raise the register pressure of the whole kernel.
            auto select_wide = [&]() {
                const int nch = (nU + 63) / 64;
                auto key_at = [&](int u) -> uint32_t { return u < nU ? ebits[u] : 0u; };
                uint32_t tau = 0u;
                bool split_ties = false;
                int need = 0, nt = 0;
                if (needSel) {
                    uint32_t lo = 0u, hi = 0x80000000u;
                    int clo = nU, chi = 0;
                    auto probe = [&](uint32_t t) -> int {
                        int cc = 0;
#pragma unroll 4
                        for (int i = 0; i < nch; ++i) cc += __popcll(__ballot(key_at(i * 64 + lane) >= t));
                        cc = __builtin_amdgcn_readfirstlane(cc);
                        if (cc >= C) {
                            lo = t;
                            clo = cc;
                        } else {
                            hi = t;
                            chi = cc;
                        }
                        return cc;
                    };
                    int cc = probe(tauPrev > 0u && tauPrev < hi ? tauPrev : 0x3f800000u);
                    uint32_t step = 1u << 18;
#pragma nounroll
                    while (cc != C && hi - lo > 2u * step) {
                        cc = probe(cc >= C ? lo + step : hi - step);
                        step = step < (1u << 28) ? step << 2 : step;
                    }
                    uint32_t wprev = 0xffffffffu;
                    int k = 0;
#pragma nounroll
                    while (cc != C && hi - lo > 1u) {
                        const uint32_t wd = hi - lo;
                        uint32_t t;
                        if ((k & 1) && wd > wprev / 2u)
                            t = lo + wd / 2u;
                        else {
                            const float frac = ((float)(clo - C) + 0.5f) * __builtin_amdgcn_rcpf((float)(clo - chi));
                            t = lo + (uint32_t)((float)wd * frac);
                            t = t <= lo ? lo + 1u : (t >= hi ? hi - 1u : t);
                            t = __builtin_amdgcn_readfirstlane(t);
                        }
                        if (!(k & 1)) wprev = wd;
                        ++k;
                        cc = probe(t);
                    }
                    tau = lo;
                    tauPrev = lo;
                    if (clo != C) {
                        int above = 0, ties = 0;
                        for (int i = 0; i < nch; ++i) {
                            const int u = i * 64 + lane;
                            const uint32_t kv = key_at(u);
                            above += __popcll(__ballot(u < nU && kv > tau));
                            ties += __popcll(__ballot(u < nU && kv == tau));
                        }
                        need = C - above;
                        split_ties = ties > need;
                        if (split_ties) {
                            for (int i = 0; i < nch; ++i) {
                                const int u = i * 64 + lane;
                                const bool tie = u < nU && key_at(u) == tau;
                                const uint64_t bm = __ballot(tie);
                                if (tie) tiep[nt + __popcll(bm & lt)] = cand_pos(u);
                                nt += __popcll(bm);
                            }
                            lds_wait();
                        }
                    }
                }
                // kept: above the threshold, or tied and among the `need` oldest tied positions
                auto kept = [&](int u) -> bool {
                    if (u >= nU) return false;
                    if (!needSel) return nU <= C;
                    const uint32_t kv = ebits[u];
                    if (kv != tau) return kv > tau;
                    if (!split_ties) return true;
                    const int p = cand_pos(u);
                    int rank = 0;
                    for (int j = 0; j < nt; ++j) rank += tiep[j] < p;
                    return rank < need;
                };
                int nF = 0;
                uint32_t kb = 0u;
                for (int i = 0; i < nch; ++i) {
                    const int u = i * 64 + lane;
                    const bool keep = kept(u);
                    const bool isF = u < nU && !keep;
                    const uint64_t bF = __ballot(isF);
                    if (isF) foldc[nF + __popcll(bF & lt)] = cand_code(u, cnt, xE0);
                    nF += __popcll(bF);
                    kb |= (uint32_t)keep << i;
                }
                kbits = kb;
                if (lane == 0) misc[5] = nF;
            };
            const int nch = (nU + 63) / 64;
            if (nch <= 2) select_compact(std::integral_constant<int, 2>{});
            else if (nch <= 5) select_compact(std::integral_constant<int, 5>{});
            else select_wide();
        } else {
            prefetch_new(nUN, cntN, ivN.xE0);
            if (needSel) snapshot(64);
        }
        lds_sync();
        const int nF = misc[5];

        // ---- fold into this block's columns: H += (phi hi + lo) v^T, s += phi hi + lo ----
        // A chunk of up to EC folded pairs is loaded to registers (every load issued
        // before any is waited for), stored to LDS transposed, then multiplied.
        constexpr int SPT = EC * (2 * F / 8) / NT;  // 16-byte pieces per thread
        const int ve1 = tid >> 2, vq4 = (tid & 3) * 4;  // EC * 4 == NT value pieces
        uint4 t4[SPT];
        uint2 t2;
        uint32_t k0 = 0u, k1 = 0u, vkeep = 0u;  // keep masks of the staged rows
        // Lane l of wave w stages pairs 2 (l % 32) and 2 (l % 32) + 1, 16-byte column
        // groups cg = 2 w + l / 32 + 2 NW m, and writes them transposed (one dword =
        // one slot of the two pairs, consecutive lanes on consecutive dwords).  Rows
        // past the chunk end load the chunk's last pair and are zeroed after the
        // store, so that every lookup and load is issued without a branch.
        constexpr int CG = SPT / 2;  // column groups per lane
        const int rp = lane & 31, cg0 = 2 * wave + (lane >> 5);
        auto stage_load = [&](int e0) {
            const int ne = nF - e0 < EC ? nF - e0 : EC;  // >= 1
            const int c0 = foldc[e0 + (2 * rp < ne ? 2 * rp : ne - 1)];
            const int c1 = foldc[e0 + (2 * rp + 1 < ne ? 2 * rp + 1 : ne - 1)];
            const int vcode = foldc[e0 + (ve1 < ne ? ve1 : ne - 1)];
            t2 = *(const uint2*)(code_v(vcode) + col0 + vq4);
            const uint16_t* p0 = code_phs(c0);
            const uint16_t* p1 = code_phs(c1);
#pragma unroll
            for (int m = 0; m < CG; ++m) {
                const int c8 = (cg0 + 2 * NW * m) * 8;
                t4[2 * m] = *(const uint4*)(p0 + c8);
                t4[2 * m + 1] = *(const uint4*)(p1 + c8);
            }
            k0 = 2 * rp < ne ? 0xffffffffu : 0u;
            k1 = 2 * rp + 1 < ne ? 0xffffffffu : 0u;
            vkeep = ve1 < ne ? 0xffffffffu : 0u;
        };
        // (the masks are applied here, so that stage_load returns with its loads in flight)
        auto stage_store = [&]() {
#pragma unroll
            for (int m = 0; m < CG; ++m) {
                const int c8 = (cg0 + 2 * NW * m) * 8;
                const uint32_t a4[4] = {t4[2 * m].x & k0, t4[2 * m].y & k0, t4[2 * m].z & k0, t4[2 * m].w & k0};
                const uint32_t b4[4] = {t4[2 * m + 1].x & k1, t4[2 * m + 1].y & k1, t4[2 * m + 1].z & k1,
                                        t4[2 * m + 1].w & k1};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t lo = (a4[j >> 1] >> (16 * (j & 1))) & 0xffffu;
                    const uint32_t hi = (b4[j >> 1] >> (16 * (j & 1))) & 0xffffu;
                    *(uint32_t*)(PR + (c8 + j) * EP + 2 * rp) = lo | (hi << 16);
                }
            }
            const uint32_t vx = t2.x & vkeep, vy = t2.y & vkeep;
            VS[(vq4 + 0) * EP + ve1] = (uint16_t)(vx & 0xffffu);
            VS[(vq4 + 1) * EP + ve1] = (uint16_t)(vx >> 16);
            VS[(vq4 + 2) * EP + ve1] = (uint16_t)(vy & 0xffffu);
            VS[(vq4 + 3) * EP + ve1] = (uint16_t)(vy >> 16);
        };
        auto fold_mma = [&]() {
            const bf16x8 ones = __builtin_bit_cast(bf16x8, u16x8{0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80,
                                                                 0x3f80, 0x3f80});
#pragma unroll
            for (int h = 0; h < HT; ++h) {
                const int ft = wave + NW * h;
                if (ft >= FT) break;  // wave-uniform
                const int pos = perm_pos(ft * 16 + r16);
                floatx4 sa = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < EC / 32; ++ks) {
                    const bf16x8 hb = *(const bf16x8*)(PR + pos * EP + ks * 32 + qg * 8);
                    const bf16x8 lb = *(const bf16x8*)(PR + (F + pos) * EP + ks * 32 + qg * 8);
                    const bf16x8 bv = *(const bf16x8*)(VS + r16 * EP + ks * 32 + qg * 8);
                    Hacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hb, bv, Hacc[h], 0, 0, 0);
                    Hacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lb, bv, Hacc[h], 0, 0, 0);
                    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hb, ones, sa, 0, 0, 0);
                    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lb, ones, sa, 0, 0, 0);
                }
                if (r16 == 0)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sP[perm_pos(ft * 16 + qg * 4 + i)] += sa[i];
            }
        };
        if (nF > 0) stage_load(0);
        if (wave == 0) slot_update();
        if (nF > 0) stage_store();
        lds_sync();  // first chunk staged, slot codes updated
        // the next interval's SRE operands, issued once the first chunk is staged (so
        // that they do not queue ahead of its loads); they arrive during the fold
        prefetch_next(nUN, cntN, ivN.xE0);
        if (nF > 0) fold_mma();
        for (int e0 = EC; e0 < nF; e0 += EC) {
            lds_sync();  // the previous chunk is consumed
            stage_load(e0);
            stage_store();
            lds_sync();
            fold_mma();
        }

        // ---- new operands of H and s ----
        if (nF > 0) {
#pragma unroll
            for (int h = 0; h < HT; ++h) {
                const int ft = wave + NW * h;
                if (ft >= FT) break;  // wave-uniform
                u16x8 hl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    hl[i] = bf16_bits(Hacc[h][i]);
                    hl[4 + i] = bf16_bits(Hacc[h][i] - bf16_val(hl[i]));
                }
                const int pos = perm_pos(ft * 16 + qg * 4);
                *(uint2*)(AX + r16 * AXS + pos) = make_uint2((uint32_t)hl[0] | ((uint32_t)hl[1] << 16),
                                                             (uint32_t)hl[2] | ((uint32_t)hl[3] << 16));
                *(uint2*)(AX + (16 + r16) * AXS + pos) = make_uint2((uint32_t)hl[4] | ((uint32_t)hl[5] << 16),
                                                                    (uint32_t)hl[6] | ((uint32_t)hl[7] << 16));
                if (r16 == 0)
#pragma unroll
                    for (int i = 0; i < 4; ++i) split3(pos + i);
            }
        }
        lds_sync();
        cnt = cntN;
    }

    // ---- state out ----
    // Cache rows replaced in this call and the window ring, in 16-byte pieces spread
    // over the chain's blocks (no block of the scan reads them from the state: the
    // call-start rows are read from the workspace copies).
    {
        constexpr int NP = D / 8;  // pieces per row
        const int nb = KW * PU, nbl = __builtin_ctz((unsigned)KW) + pl, rank = jw + KW * ju;
        const int nrc = cnt > rank ? (cnt - rank + nb - 1) >> nbl : 0;  // this block's cache rows
        for (int q = tid; q < nrc * NP; q += NT) {
            const int i = rank + nb * (q / NP), pc = (q % NP) * 8, code = cref[i];
            if (code >= 0) {
                const uint4 k4 = *(const uint4*)(xrow_k<bf16>(a, chain, b, g, code) + pc);
                const uint4 v4 = *(const uint4*)(xrow_v<bf16>(a, chain, b, g, code) + pc);
                *(uint4*)(ch.cache_k<bf16>() + (size_t)i * D + pc) = k4;
                *(uint4*)(ch.cache_v<bf16>() + (size_t)i * D + pc) = v4;
            }
        }
        // and their z = W k, from which a decode step recomputes the features
        constexpr int ZP = F / 2 / 4;
        for (int q = tid; q < nrc * ZP; q += NT) {
            const int i = rank + nb * (q / ZP), pc = (q % ZP) * 4, code = cref[i];
            if (code >= 0) *(float4*)(ch.cz() + (size_t)i * (F / 2) + pc) = *(const float4*)(ws_zX(a, chain, code) + pc);
        }
        if (w > 0) {
            const int64_t tend = t0 + ns;
            const int64_t p0 = tend - w > t0 ? tend - w : t0;
            const int nr = (int)(tend - p0);
            const int nrr = nr > rank ? (nr - rank + nb - 1) >> nbl : 0;
            for (int q = tid; q < nrr * NP; q += NT) {
                const int i = rank + nb * (q / NP), pc = (q % NP) * 8;
                const int64_t p = p0 + i;
                const int slot = (int)(p % w);
                const size_t src = (((size_t)b * n + (size_t)(p - t0)) * d.Hkv + g) * D + pc;
                const uint4 k4 = *(const uint4*)((const bf16*)a.k + src);
                const uint4 v4 = *(const uint4*)((const bf16*)a.v + src);
                *(uint4*)(ch.ring_k<bf16>() + (size_t)slot * D + pc) = k4;
                *(uint4*)(ch.ring_v<bf16>() + (size_t)slot * D + pc) = v4;
            }
        }
    }
    // this column slice's rows of H^T (lead blocks); block 0 also s, positions, counts.
    // Every block of the chain reads H, s, the count and the positions at its start;
    // with no exchange in a call (no cache, or no interval that must select) nothing
    // else orders a late-starting block's reads before these stores, so each lead block
    // first waits until all KW * PU blocks have counted their reads in xsync[2].
    if (!lead) return;
    if (tid == 0) {
        uint32_t polls = 0;
        while (__hip_atomic_load(&xsync[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)(KW * PU)) {
            if (__hip_atomic_load(&xsync[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u || ++polls > kSpinLimit) {
                __hip_atomic_store(&xsync[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&((StateHeader*)a.state)->fault, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    lds_sync();
#pragma unroll
    for (int h = 0; h < HT; ++h) {
        const int ft = wave + NW * h;
        if (ft < FT)
            *(float4*)(ch.H() + (size_t)(col0 + r16) * F + ft * 16 + qg * 4) =
                make_float4(Hacc[h][0], Hacc[h][1], Hacc[h][2], Hacc[h][3]);
    }
    if (jw != 0) return;
    for (int i = tid; i < F; i += NT) ch.s()[i] = sP[perm_pos(i)];
    for (int i = tid; i < cnt; i += NT) ch.cpos()[i] = cpos[i];
    if (tid == 0) {
        ch.cnt() = cnt;
        ch.tok() = t0 + ns;
        ch.incv() = 0;  // stored incremental decode scores no longer match
    }
}

}  // namespace lola
