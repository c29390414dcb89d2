// Prefill kernels of the LoLA layer (gfx950).
//
// One lola_prefill_chunk call runs three launches on the caller's stream:
//   1. prologue  -- feature rows phi(k) for the window keys at the call start
//                   and the new keys; copies of the window ring and the cache
//                   as they stand at the call start (the scan rewrites them).
//   2. scan      -- one workgroup per (sequence, KV head) chain walks the
//                   update intervals in order: snapshot (H, s, cache) at the
//                   interval start, SRE of cache + leaving keys, top-C keep,
//                   outer-product fold of the rest, slot update.  This is the
//                   serial recurrence of the method.
//   3. output    -- fully parallel over (interval, chain, query tile): exact
//                   softmax over window + cache keys, linear read of the
//                   snapshot state and of keys that left the window inside
//                   the interval, one shared denominator.
//
// Method: LoLA technical summary (gist.science), sections "Het Self-Recall
// Error (SRE) Mechanisme" (SRE equation) and "Inferentiestrategie" (per
// interval: score leaving + cached pairs, keep the highest, fold the lowest by
// outer products, combine linear + cache + window attention).
#pragma once

#include "lola_internal.h"

namespace lola {

// ---------------------------------------------------------------------------
// addressing helpers
// ---------------------------------------------------------------------------
struct Chain {
    unsigned char* base;
    const StateLayout* sl;
    __device__ int64_t& tok() const { return *(int64_t*)(base + sl->otok); }
    __device__ int32_t& cnt() const { return *(int32_t*)(base + sl->ocnt); }
    __device__ float* H() const { return (float*)(base + sl->oH); }
    __device__ float* s() const { return (float*)(base + sl->os); }
    __device__ int32_t* cpos() const { return (int32_t*)(base + sl->ocpos); }
    template <typename T> __device__ T* ring_k() const { return (T*)(base + sl->oring_k); }
    template <typename T> __device__ T* ring_v() const { return (T*)(base + sl->oring_v); }
    template <typename T> __device__ T* cache_k() const { return (T*)(base + sl->ocache_k); }
    template <typename T> __device__ T* cache_v() const { return (T*)(base + sl->ocache_v); }
};

__device__ __forceinline__ Chain chain_of(const Args& a, int chain)
{
    Chain c;
    c.base = a.state + a.sl.chains + (size_t)chain * a.sl.chain_bytes;
    c.sl = &a.sl;
    return c;
}

// Rows of the extended sequence X of one chain: x < w is the window as it
// stood at the call start (position t0 - w + x, copied to the workspace),
// x >= w is new token x - w of this call.
template <typename T>
__device__ __forceinline__ const T* xrow_k(const Args& a, int chain, int b, int g, int x)
{
    if (x < a.d.w) return (const T*)(a.ws + a.wl.ring0_k) + ((size_t)chain * a.d.w + x) * a.d.D;
    return (const T*)a.k + (((size_t)b * a.n + (x - a.d.w)) * a.d.Hkv + g) * a.d.D;
}
template <typename T>
__device__ __forceinline__ const T* xrow_v(const Args& a, int chain, int b, int g, int x)
{
    if (x < a.d.w) return (const T*)(a.ws + a.wl.ring0_v) + ((size_t)chain * a.d.w + x) * a.d.D;
    return (const T*)a.v + (((size_t)b * a.n + (x - a.d.w)) * a.d.Hkv + g) * a.d.D;
}
// Cache references: ref >= 0 is an X row, ref < 0 is call-start cache slot -ref-1.
template <typename T>
__device__ __forceinline__ const T* ref_k(const Args& a, int chain, int b, int g, int ref)
{
    if (ref >= 0) return xrow_k<T>(a, chain, b, g, ref);
    int Cp = a.d.C > 0 ? a.d.C : 1;
    return (const T*)(a.ws + a.wl.cache0_k) + ((size_t)chain * Cp + (-ref - 1)) * a.d.D;
}
template <typename T>
__device__ __forceinline__ const T* ref_v(const Args& a, int chain, int b, int g, int ref)
{
    if (ref >= 0) return xrow_v<T>(a, chain, b, g, ref);
    int Cp = a.d.C > 0 ? a.d.C : 1;
    return (const T*)(a.ws + a.wl.cache0_v) + ((size_t)chain * Cp + (-ref - 1)) * a.d.D;
}

__device__ __forceinline__ int64_t ws_t0(const Args& a, int b) { return ((const int64_t*)(a.ws + a.wl.t0))[b]; }
__device__ __forceinline__ float* ws_phiX(const Args& a, int chain, int x)
{
    return (float*)(a.ws + a.wl.phiX) + ((size_t)chain * a.wl.X + x) * a.d.F;
}
__device__ __forceinline__ float* ws_cphi(const Args& a, int chain, int slot)
{
    int Cp = a.d.C > 0 ? a.d.C : 1;
    return (float*)(a.ws + a.wl.cphi) + ((size_t)chain * Cp + slot) * a.d.F;
}

// ---------------------------------------------------------------------------
// 1. prologue: phi rows + call-start copies.  grid (ceil((X + C) / 64), B*Hkv)
//    block 256: each wave handles 16 rows; W of the chain's head sits in LDS.
// ---------------------------------------------------------------------------
template <int D, int Fh, typename T>
__global__ __launch_bounds__(256) void prologue_kernel(Args a)
{
    constexpr int RPW = 16;  // rows per wave
    __shared__ float Ws[Fh][D + 1];
    __shared__ float xs[4][D];
    const int chain = blockIdx.y, b = chain / a.d.Hkv, g = chain % a.d.Hkv;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int w = a.d.w, C = a.d.C, X = a.wl.X;
    Chain ch = chain_of(a, chain);
    const int64_t t0 = ch.tok();
    const int cnt0 = min(max(ch.cnt(), 0), C);
    const float* W = (const float*)(a.state + a.sl.W) + (size_t)g * Fh * D;
    for (int i = threadIdx.x; i < Fh * D; i += 256) Ws[i / D][i % D] = W[i];
    if (blockIdx.x == 0 && threadIdx.x == 0 && g == 0) ((int64_t*)(a.ws + a.wl.t0))[b] = t0;

    for (int rr = 0; rr < RPW; ++rr) {
        const int row = (blockIdx.x * 4 + wave) * RPW + rr;
        const T* src = nullptr;
        const T* srcv = nullptr;
        T* cpk = nullptr;
        T* cpv = nullptr;
        float* phi_out = nullptr;
        if (row < X) {
            phi_out = ws_phiX(a, chain, row);
            if (row < w) {
                int64_t p = t0 - w + row;
                cpk = (T*)(a.ws + a.wl.ring0_k) + ((size_t)chain * w + row) * D;
                cpv = (T*)(a.ws + a.wl.ring0_v) + ((size_t)chain * w + row) * D;
                if (p >= 0) {
                    int slot = (int)(p % w);
                    src = ch.ring_k<T>() + (size_t)slot * D;
                    srcv = ch.ring_v<T>() + (size_t)slot * D;
                }
            } else {
                src = (const T*)a.k + (((size_t)b * a.n + (row - w)) * a.d.Hkv + g) * D;
            }
        } else if (row < X + C) {
            int i = row - X;
            phi_out = ws_cphi(a, chain, i);
            int Cp = C > 0 ? C : 1;
            cpk = (T*)(a.ws + a.wl.cache0_k) + ((size_t)chain * Cp + i) * D;
            cpv = (T*)(a.ws + a.wl.cache0_v) + ((size_t)chain * Cp + i) * D;
            if (i < cnt0) {
                src = ch.cache_k<T>() + (size_t)i * D;
                srcv = ch.cache_v<T>() + (size_t)i * D;
            }
        }
        // stage the key row; copy raw key/value rows that the scan will overwrite
        __syncthreads();
        for (int j = lane; j < D; j += 64) {
            float x = src ? to_f32(src[j]) : 0.f;
            xs[wave][j] = x;
            if (cpk) {
                cpk[j] = src ? src[j] : from_f32<T>(0.f);
                cpv[j] = srcv ? srcv[j] : from_f32<T>(0.f);
            }
        }
        __syncthreads();
        if (!phi_out) continue;
        float z = 0.f;
        if (lane < Fh) {
#pragma unroll 8
            for (int j = 0; j < D; ++j) z += Ws[lane][j] * xs[wave][j];
        }
        // phi = [softmax(z); softmax(-z)] over the Fh lanes
        float zmax = wave_max(lane < Fh ? z : -INFINITY);
        float zmin = -wave_max(lane < Fh ? -z : -INFINITY);
        float ep = lane < Fh ? expf(z - zmax) : 0.f;
        float en = lane < Fh ? expf(zmin - z) : 0.f;
        float sp = wave_sum(ep), sn = wave_sum(en);
        if (lane < Fh) {
            bool valid = src != nullptr;
            phi_out[lane] = valid ? ep / sp : 0.f;
            phi_out[Fh + lane] = valid ? en / sn : 0.f;
        }
    }
}

// ---------------------------------------------------------------------------
// 2. scan: one workgroup per chain, intervals in order.
// ---------------------------------------------------------------------------
struct ScanSmem {
    // byte offsets into dynamic LDS
    size_t H, s, esc, upos, keep, cref, cpos, fold, freed, keptE, misc, total;
};

__host__ __device__ inline ScanSmem scan_smem(int D, int F, int C, int L)
{
    ScanSmem m;
    int U = C + L;
    int Cp = C > 0 ? C : 1;
    size_t off = 0;
    m.H = off;     off += sizeof(float) * (size_t)F * (D + 4);
    m.s = off;     off += sizeof(float) * F;
    m.esc = off;   off += sizeof(float) * U;
    m.upos = off;  off += sizeof(int) * U;
    m.keep = off;  off += sizeof(int) * U;
    m.cref = off;  off += sizeof(int) * Cp;
    m.cpos = off;  off += sizeof(int) * Cp;
    m.fold = off;  off += sizeof(int) * U;
    m.freed = off; off += sizeof(int) * Cp;
    m.keptE = off; off += sizeof(int) * (L + 1);
    m.misc = off;  off += sizeof(int) * 8;
    m.total = align_up(off, 16);
    return m;
}

template <int D, int F, typename T>
__global__ __launch_bounds__(256) void scan_kernel(Args a)
{
    constexpr int NW = 4, HP = D + 4;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const Dims& d = a.d;
    const int w = d.w, C = d.C, L = d.L;
    const ScanSmem sm = scan_smem(D, F, C, L);
    float* Hs = (float*)(smem + sm.H);
    float* ss = (float*)(smem + sm.s);
    float* esc = (float*)(smem + sm.esc);
    int* upos = (int*)(smem + sm.upos);
    int* keep = (int*)(smem + sm.keep);
    int* cref = (int*)(smem + sm.cref);
    int* cpos = (int*)(smem + sm.cpos);
    int* fold = (int*)(smem + sm.fold);
    int* freed = (int*)(smem + sm.freed);
    int* keptE = (int*)(smem + sm.keptE);
    int* misc = (int*)(smem + sm.misc);

    const int chain = blockIdx.x, b = chain / d.Hkv, g = chain % d.Hkv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, qg = lane >> 4;
    Chain ch = chain_of(a, chain);
    const int64_t t0 = ws_t0(a, b);
    const int n = a.n, NI = a.NI, X = a.wl.X;
    const int Cp = C > 0 ? C : 1;

    // load the state of this chain
    for (int i = tid; i < F * D; i += 256) Hs[(i / D) * HP + (i % D)] = ch.H()[i];
    for (int i = tid; i < F; i += 256) ss[i] = ch.s()[i];
    int cnt = min(max(ch.cnt(), 0), C);
    for (int i = tid; i < cnt; i += 256) {
        cpos[i] = ch.cpos()[i];
        cref[i] = -(i + 1);
    }
    __syncthreads();

    float* snapH = (float*)(a.ws + a.wl.snapH) + (size_t)chain * NI * F * D;
    float* snapS = (float*)(a.ws + a.wl.snapS) + (size_t)chain * NI * F;
    int* snapRef = (int*)(a.ws + a.wl.snapRef) + (size_t)chain * NI * Cp;
    int* snapN = (int*)(a.ws + a.wl.snapN) + (size_t)chain * NI;

    for (int c = 0; c < NI; ++c) {
        const int64_t ap = t0 + (int64_t)c * L;
        const int64_t ep = ap + L < t0 + n ? ap + L : t0 + n;

        // ---- interval-start snapshot for the output pass ----
        {
            float* dst = snapH + (size_t)c * F * D;
            for (int i = tid; i < F * D / 4; i += 256) {
                int f = (i * 4) / D, col = (i * 4) % D;
                *(float4*)(dst + (size_t)f * D + col) = *(const float4*)(Hs + f * HP + col);
            }
            for (int i = tid; i < F; i += 256) snapS[(size_t)c * F + i] = ss[i];
            for (int i = tid; i < cnt; i += 256) snapRef[(size_t)c * Cp + i] = cref[i];
            if (tid == 0) snapN[c] = cnt;
        }

        // ---- candidates: cache slots [0, cnt) then leaving keys ----
        const int64_t eS = ap - w > 0 ? ap - w : 0;
        const int64_t eE = ep - w;  // exclusive
        const int nE = eE > eS ? (int)(eE - eS) : 0;
        const int nU = cnt + nE;
        const int xE0 = (int)(eS - (t0 - w));  // X row of the first leaving key
        for (int u = tid; u < nU; u += 256) upos[u] = u < cnt ? cpos[u] : (int)(eS + (u - cnt));

        auto cand_phi = [&](int u) -> const float* {
            return u < cnt ? ws_cphi(a, chain, u) : ws_phiX(a, chain, xE0 + (u - cnt));
        };
        auto cand_v = [&](int u) -> const T* {
            return u < cnt ? ref_v<T>(a, chain, b, g, cref[u]) : xrow_v<T>(a, chain, b, g, xE0 + (u - cnt));
        };
        __syncthreads();

        // ---- SRE of every candidate against the interval-start state ----
        // n^T tile: acc[ct] = phi(k_u) . H[:, 16ct + r16] for 16 candidates per
        // tile (f32 MFMA, exact fp32 products); d_u = phi(k_u) . s.
        for (int tile = wave; tile * 16 < nU; tile += NW) {
            const int u = tile * 16 + r16;
            float av[F / 4];
            if (u < nU) {
                const float* ph = cand_phi(u) + qg * (F / 4);
#pragma unroll
                for (int m = 0; m < F / 4; m += 4) {
                    float4 t4 = *(const float4*)(ph + m);
                    av[m] = t4.x; av[m + 1] = t4.y; av[m + 2] = t4.z; av[m + 3] = t4.w;
                }
            } else {
#pragma unroll
                for (int m = 0; m < F / 4; ++m) av[m] = 0.f;
            }
            floatx4 acc[D / 16];
#pragma unroll
            for (int ct = 0; ct < D / 16; ++ct) acc[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
            float dpart = 0.f;
#pragma unroll 4
            for (int m = 0; m < F / 4; ++m) {
                const int f = qg * (F / 4) + m;
                dpart += av[m] * ss[f];
#pragma unroll
                for (int ct = 0; ct < D / 16; ++ct)
                    acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[m], Hs[f * HP + ct * 16 + r16], acc[ct], 0, 0, 0);
            }
            dpart += __shfl_xor(dpart, 16, 64);
            dpart += __shfl_xor(dpart, 32, 64);
            float err[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = qg * 4 + i;
                const int uu = tile * 16 + row;
                const float drow = __shfl(dpart, row, 64);
                const T* vr = uu < nU ? cand_v(uu) : nullptr;
                float e = 0.f;
#pragma unroll
                for (int ct = 0; ct < D / 16; ++ct) {
                    float r = drow > 0.f ? acc[ct][i] / drow : 0.f;
                    float vv = vr ? to_f32(vr[ct * 16 + r16]) : 0.f;
                    float df = r - vv;
                    e += df * df;
                }
                err[i] = e;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float e = err[i];
                e += __shfl_xor(e, 1, 64);
                e += __shfl_xor(e, 2, 64);
                e += __shfl_xor(e, 4, 64);
                e += __shfl_xor(e, 8, 64);
                const int uu = tile * 16 + qg * 4 + i;
                if (r16 == 0 && uu < nU) esc[uu] = e;
            }
        }
        __syncthreads();

        // ---- keep the C highest by (SRE desc, position asc) ----
        for (int u = tid; u < nU; u += 256) {
            int kp = 1;
            if (nU > C) {
                const uint32_t eu = __float_as_uint(esc[u]);
                const int pu = upos[u];
                int rank = 0;
                for (int v2 = 0; v2 < nU; ++v2) {
                    const uint32_t ev = __float_as_uint(esc[v2]);
                    rank += (ev > eu) || (ev == eu && upos[v2] < pu);
                }
                kp = rank < C;
            }
            keep[u] = kp;
        }
        __syncthreads();

        // ---- compaction (wave 0): fold list, freed slots, kept leaving keys ----
        if (wave == 0) {
            int nF = 0, nFr = 0, nK = 0;
            const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
            for (int base = 0; base < nU; base += 64) {
                const int u = base + lane;
                const bool valid = u < nU;
                const bool kp = valid && keep[u];
                const bool isF = valid && !kp;
                const bool isFr = valid && u < cnt && !kp;
                const bool isK = valid && u >= cnt && kp;
                const uint64_t bF = __ballot(isF), bFr = __ballot(isFr), bK = __ballot(isK);
                if (isF) fold[nF + __popcll(bF & lt)] = u;
                if (isFr) freed[nFr + __popcll(bFr & lt)] = u;
                if (isK) keptE[nK + __popcll(bK & lt)] = u;
                nF += __popcll(bF);
                nFr += __popcll(bFr);
                nK += __popcll(bK);
            }
            if (lane == 0) { misc[0] = nF; misc[1] = nFr; misc[2] = nK; }
        }
        __syncthreads();
        const int nF = misc[0], nFr = misc[1], nK = misc[2];

        // ---- fold: H += sum_f phi(k_f) v_f^T, s += sum_f phi(k_f) ----
        for (int ft = wave; ft < F / 16; ft += NW) {
            floatx4 acc[D / 16];
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[dt][i] = Hs[(ft * 16 + qg * 4 + i) * HP + dt * 16 + r16];
            for (int kk = 0; kk < nF; kk += 4) {
                const int kx = kk + qg;
                float av = 0.f;
                const T* vr = nullptr;
                if (kx < nF) {
                    const int u = fold[kx];
                    av = cand_phi(u)[ft * 16 + r16];
                    vr = cand_v(u);
                }
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) {
                    float bv = vr ? to_f32(vr[dt * 16 + r16]) : 0.f;
                    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[dt], 0, 0, 0);
                }
            }
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) Hs[(ft * 16 + qg * 4 + i) * HP + dt * 16 + r16] = acc[dt][i];
        }
        for (int f = tid; f < F; f += 256) {
            float acc = ss[f];
            for (int kx = 0; kx < nF; ++kx) acc += cand_phi(fold[kx])[f];
            ss[f] = acc;
        }
        __syncthreads();

        // ---- kept leaving keys take the freed slots, then new slots ----
        for (int i = tid; i < nK; i += 256) {
            const int u = keptE[i];
            const int slot = i < nFr ? freed[i] : cnt + (i - nFr);
            const int x = xE0 + (u - cnt);
            cref[slot] = x;
            cpos[slot] = upos[u];
        }
        for (int idx = tid; idx < nK * F; idx += 256) {
            const int i = idx / F, f = idx % F;
            const int u = keptE[i];
            const int slot = i < nFr ? freed[i] : cnt + (i - nFr);
            ws_cphi(a, chain, slot)[f] = ws_phiX(a, chain, xE0 + (u - cnt))[f];
        }
        cnt = nU < C ? nU : C;
        __syncthreads();
    }

    // ---- write the chain's state back ----
    for (int i = tid; i < F * D; i += 256) ch.H()[i] = Hs[(i / D) * HP + (i % D)];
    for (int i = tid; i < F; i += 256) ch.s()[i] = ss[i];
    for (int i = tid; i < cnt; i += 256) ch.cpos()[i] = cpos[i];
    for (int idx = tid; idx < cnt * D; idx += 256) {
        const int i = idx / D, j = idx % D;
        if (cref[i] >= 0) {
            ch.cache_k<T>()[(size_t)i * D + j] = xrow_k<T>(a, chain, b, g, cref[i])[j];
            ch.cache_v<T>()[(size_t)i * D + j] = xrow_v<T>(a, chain, b, g, cref[i])[j];
        }
    }
    if (w > 0) {
        const int64_t tend = t0 + n;
        const int64_t p0 = tend - w > t0 ? tend - w : t0;
        const int nr = (int)(tend - p0);
        for (int idx = tid; idx < nr * D; idx += 256) {
            const int i = idx / D, j = idx % D;
            const int64_t p = p0 + i;
            const int slot = (int)(p % w);
            const size_t src = (((size_t)b * n + (size_t)(p - t0)) * d.Hkv + g) * D + j;
            ch.ring_k<T>()[(size_t)slot * D + j] = ((const T*)a.k)[src];
            ch.ring_v<T>()[(size_t)slot * D + j] = ((const T*)a.v)[src];
        }
    }
    if (tid == 0) {
        ch.cnt() = cnt;
        ch.tok() = t0 + n;
    }
}

// ---------------------------------------------------------------------------
// 3. output pass.  grid (NI * ceil(G*L/64), B*Hkv), block 256 (4 waves x 16
//    query rows).  Query row r of an interval is (head g*G + r/L, token r%L).
//    Per wave everything is a 16-column tile over the wave's queries:
//      z^T   = W . Q^T            -> phi(q) (held per lane, feature map)
//      O^T   = H_c^T . phi(q)^T   (linear read of the snapshot state)
//      per 32-key block: S^T = K . Q^T, kappa^T = phi(K) . phi(q)^T,
//      online softmax with running max M >= 0, O^T += V^T . P^T.
//    bf16 io uses bf16 MFMA (W split hi+lo for z); f32 io uses f32 MFMA.
// ---------------------------------------------------------------------------
template <int Fh>
__device__ __forceinline__ int held_feature(int qg, int hi)
{
    // feature index of held value hi (0 .. Fh/2-1) in lane group qg
    constexpr int H4 = Fh / 4;
    const int part = hi < H4 ? 0 : Fh;
    const int h = hi < H4 ? hi : hi - H4;
    return part + (h >> 2) * 16 + qg * 4 + (h & 3);
}

template <int D, int F, typename T>
__global__ __launch_bounds__(256) void output_kernel(Args a)
{
    using M = Mma<T>;
    constexpr int KPL = M::KPL;
    constexpr int Fh = F / 2;
    constexpr int QM = D / (4 * KPL);     // MFMAs per D contraction
    constexpr int FM = (F / 4) / KPL;     // MFMAs per F contraction
    constexpr int NH = F / 4;             // feature values held per lane
    const Dims& d = a.d;
    const int G = d.G, L = d.L, w = d.w;
    const int chain = blockIdx.y, b = chain / d.Hkv, g = chain % d.Hkv;
    const int rows = G * L;
    const int wpi = (rows + 63) / 64;
    const int c = blockIdx.x / wpi, rblk = blockIdx.x % wpi;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15, qg = lane >> 4;
    const int64_t t0 = ws_t0(a, b);
    const int64_t ap = t0 + (int64_t)c * L;
    const int64_t ep = ap + L < t0 + a.n ? ap + L : t0 + a.n;
    const int Lc = (int)(ep - ap);
    if (rblk * 64 + wave * 16 >= rows) return;  // whole wave idle (no block-level sync below)

    const int r = rblk * 64 + wave * 16 + r16;
    const int hl = r / L, ti = r % L;
    const bool qvalid = r < rows && ti < Lc;
    const int h = g * G + (qvalid ? hl : 0);
    const int64_t t = qvalid ? ap + ti : -1;

    // ---- Q^T fragments: slot (qg*KPL + j) of MFMA m <-> d = qg*D/4 + m*KPL + j ----
    typename M::frag qf[QM];
    {
        const T* qp = (const T*)a.q + (((size_t)b * a.n + (size_t)(qvalid ? ap + ti - t0 : 0)) * d.Hq + h) * D + qg * (D / 4);
#pragma unroll
        for (int m = 0; m < QM; ++m) {
            float tmp[KPL];
#pragma unroll
            for (int j = 0; j < KPL; ++j) tmp[j] = qvalid ? to_f32(qp[m * KPL + j]) : 0.f;
            qf[m] = M::pack(tmp);
        }
    }

    // ---- phi(q): z^T = W . Q^T, W rows as A (bf16: hi + lo split) ----
    float hq[NH];
    {
        const float* W = (const float*)(a.state + a.sl.W) + (size_t)g * Fh * D;
        floatx4 zt[Fh / 16];
#pragma unroll
        for (int ft = 0; ft < Fh / 16; ++ft) {
            zt[ft] = floatx4{0.f, 0.f, 0.f, 0.f};
            const float* wr = W + (size_t)(ft * 16 + r16) * D + qg * (D / 4);
#pragma unroll
            for (int m = 0; m < QM; ++m) {
                float hi[KPL], lo[KPL];
#pragma unroll
                for (int j = 0; j < KPL; ++j) {
                    float x = wr[m * KPL + j];
                    if constexpr (KPL == 1) {
                        hi[j] = x;
                        lo[j] = 0.f;
                    } else {
                        float xh = to_f32(from_f32<bf16>(x));
                        hi[j] = xh;
                        lo[j] = x - xh;
                    }
                }
                zt[ft] = M::mma(M::pack(hi), qf[m], zt[ft]);
                if constexpr (KPL > 1) zt[ft] = M::mma(M::pack(lo), qf[m], zt[ft]);
            }
        }
        // lane holds z[feature ft*16 + qg*4 + i] of query r16
        float zmax = -INFINITY, zmin = INFINITY;
#pragma unroll
        for (int ft = 0; ft < Fh / 16; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                zmax = fmaxf(zmax, zt[ft][i]);
                zmin = fminf(zmin, zt[ft][i]);
            }
        zmax = fmaxf(zmax, __shfl_xor(zmax, 16, 64));
        zmax = fmaxf(zmax, __shfl_xor(zmax, 32, 64));
        zmin = fminf(zmin, __shfl_xor(zmin, 16, 64));
        zmin = fminf(zmin, __shfl_xor(zmin, 32, 64));
        float sp = 0.f, sn = 0.f;
#pragma unroll
        for (int ft = 0; ft < Fh / 16; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float ep_ = expf(zt[ft][i] - zmax), en_ = expf(zmin - zt[ft][i]);
                hq[ft * 4 + i] = ep_;
                hq[Fh / 4 + ft * 4 + i] = en_;
                sp += ep_;
                sn += en_;
            }
        sp += __shfl_xor(sp, 16, 64);
        sp += __shfl_xor(sp, 32, 64);
        sn += __shfl_xor(sn, 16, 64);
        sn += __shfl_xor(sn, 32, 64);
#pragma unroll
        for (int j = 0; j < NH / 2; ++j) {
            hq[j] /= sp;
            hq[NH / 2 + j] /= sn;
        }
    }
    typename M::frag pf[FM];
#pragma unroll
    for (int mf = 0; mf < FM; ++mf) pf[mf] = M::pack(hq + mf * KPL);

    // ---- linear read of the snapshot: O^T = H_c^T phi(q)^T, Z = s_c . phi(q) ----
    const int NI = a.NI;
    const float* sH = (const float*)(a.ws + a.wl.snapH) + ((size_t)chain * NI + c) * F * D;
    const float* sS = (const float*)(a.ws + a.wl.snapS) + ((size_t)chain * NI + c) * F;
    floatx4 O[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        O[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mf = 0; mf < FM; ++mf) {
            float tmp[KPL];
#pragma unroll
            for (int j = 0; j < KPL; ++j) tmp[j] = sH[(size_t)held_feature<Fh>(qg, mf * KPL + j) * D + dt * 16 + r16];
            O[dt] = M::mma(M::pack(tmp), pf[mf], O[dt]);
        }
    }
    float zl = 0.f;
#pragma unroll
    for (int j = 0; j < NH; ++j) zl += hq[j] * sS[held_feature<Fh>(qg, j)];
    zl += __shfl_xor(zl, 16, 64);
    zl += __shfl_xor(zl, 32, 64);
    float Zp = qg == 0 ? zl : 0.f;  // per-lane partial of the denominator
    float mrun = 0.f;               // running max, floored at 0 (linear terms carry e^-M)

    // ---- keys: span positions [sp0, ep) then the snapshot cache ----
    const int Cp = d.C > 0 ? d.C : 1;
    const int64_t sp0 = ap - w > 0 ? ap - w : 0;
    const int nSpan = (int)(ep - sp0);
    const int ccnt = ((const int*)(a.ws + a.wl.snapN))[(size_t)chain * NI + c];
    const int* sref = (const int*)(a.ws + a.wl.snapRef) + ((size_t)chain * NI + c) * Cp;
    const int nK = nSpan + ccnt;
    const int xs0 = (int)(sp0 - (t0 - w));
    const float tau = d.tau;
    const int64_t lastPend = ep - 1 - w;  // keys at or before this are pending for some query

    auto key_k = [&](int kidx) -> const T* {
        return kidx < nSpan ? xrow_k<T>(a, chain, b, g, xs0 + kidx) : ref_k<T>(a, chain, b, g, sref[kidx - nSpan]);
    };
    auto key_v = [&](int kidx) -> const T* {
        return kidx < nSpan ? xrow_v<T>(a, chain, b, g, xs0 + kidx) : ref_v<T>(a, chain, b, g, sref[kidx - nSpan]);
    };

    for (int base = 0; base < nK; base += 32) {
        floatx4 sT[2], kT[2];
        const bool anyPend = base < nSpan && sp0 + base <= lastPend;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int kr = base + tt * 16 + r16;  // A-operand row (key) of this lane
            const bool kv = kr < nK;
            const T* kp = key_k(kv ? kr : 0) + qg * (D / 4);
            sT[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < QM; ++m) {
                float tmp[KPL];
#pragma unroll
                for (int j = 0; j < KPL; ++j) tmp[j] = kv ? to_f32(kp[m * KPL + j]) : 0.f;
                sT[tt] = M::mma(M::pack(tmp), qf[m], sT[tt]);
            }
            kT[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (anyPend) {
                const bool sv = kr < nSpan;
                const float* php = ws_phiX(a, chain, xs0 + (sv ? kr : 0));
#pragma unroll
                for (int mf = 0; mf < FM; ++mf) {
                    float tmp[KPL];
#pragma unroll
                    for (int j = 0; j < KPL; ++j) tmp[j] = sv ? php[held_feature<Fh>(qg, mf * KPL + j)] : 0.f;
                    kT[tt] = M::mma(M::pack(tmp), pf[mf], kT[tt]);
                }
            }
        }
        // classify the lane's 8 keys for its query and find the block max
        float lg[8];
        int kind[8];  // 0 none, 1 softmax, 2 pending (linear)
        float bmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int tt = j >> 2, i = j & 3;
            const int kidx = base + tt * 16 + qg * 4 + i;
            int kd = 0;
            if (qvalid && kidx < nK) {
                if (kidx < nSpan) {
                    const int64_t p = sp0 + kidx;
                    if (p <= t) kd = (p >= t - w + 1) ? 1 : 2;
                } else {
                    kd = 1;
                }
            }
            kind[j] = kd;
            lg[j] = tau * sT[tt][i];
            if (kd == 1) bmax = fmaxf(bmax, lg[j]);
        }
        bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
        const float mnew = fmaxf(mrun, bmax);
        const float resc = expf(mrun - mnew);
        mrun = mnew;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) O[dt] *= resc;
        Zp *= resc;
        const float elin = expf(-mrun);
        float p8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int tt = j >> 2, i = j & 3;
            float pv = 0.f;
            if (kind[j] == 1) pv = expf(lg[j] - mrun);
            else if (kind[j] == 2) pv = kT[tt][i] * elin;
            p8[j] = pv;
            Zp += pv;
        }
        // O^T += V^T P^T: slot (qg*KPL + jj) of MFMA mi <-> the lane's key j = mi*KPL + jj
        const T* vrow[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int kidx = base + (j >> 2) * 16 + qg * 4 + (j & 3);
            vrow[j] = kidx < nK ? key_v(kidx) : nullptr;
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
            for (int mi = 0; mi < 8 / KPL; ++mi) {
                float va[KPL];
#pragma unroll
                for (int jj = 0; jj < KPL; ++jj) {
                    const T* vr = vrow[mi * KPL + jj];
                    va[jj] = vr ? to_f32(vr[dt * 16 + r16]) : 0.f;
                }
                O[dt] = M::mma(M::pack(va), M::pack(p8 + mi * KPL), O[dt]);
            }
        }
    }

    // ---- finish: shared denominator, store o[t][h][d] ----
    float Z = Zp;
    Z += __shfl_xor(Z, 16, 64);
    Z += __shfl_xor(Z, 32, 64);
    if (qvalid) {
        T* op = (T*)a.out + (((size_t)b * a.n + (size_t)(t - t0)) * d.Hq + h) * D;
        const float inv = 1.f / Z;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) op[dt * 16 + qg * 4 + i] = from_f32<T>(O[dt][i] * inv);
    }
}

}  // namespace lola
