// Prefill kernels of the LoLA layer (gfx950).
//
// One lola_prefill_chunk call runs three launches on the caller's stream:
//   1. prologue  -- feature rows phi(k) for the window keys at the call start
//                   and the new keys (and, bf16 io, their z = W k for the
//                   state's cache); copies of the window ring and the cache
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

#include <type_traits>

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
    __device__ float* cz() const { return (float*)(base + sl->ocz); }  // bf16 io: [C][Fh]
    __device__ float* cscore() const { return (float*)(base + sl->oscore); }
    __device__ int32_t& incv() const { return *(int32_t*)(base + sl->oincv); }  // incremental n, d valid
    __device__ float* cn() const { return (float*)(base + sl->ocn); }           // [C][D]
    __device__ float* cd() const { return (float*)(base + sl->ocd); }           // [C]
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
// bf16 hi/lo split rows of phi (2F values: hi parts, then lo parts), features
// permuted so that an MFMA operand lane reads 8 contiguous values.
__device__ __forceinline__ uint16_t* ws_phiS(const Args& a, int chain, int x)
{
    return (uint16_t*)(a.ws + a.wl.phiS) + ((size_t)chain * a.wl.X + x) * 2 * a.d.F;
}
__device__ __forceinline__ uint16_t* ws_cphiS(const Args& a, int chain, int slot)
{
    int Cp = a.d.C > 0 ? a.d.C : 1;
    return (uint16_t*)(a.ws + a.wl.cphiS) + ((size_t)chain * Cp + slot) * 2 * a.d.F;
}
// z = W k of extended row x (bf16 io), natural feature order
__device__ __forceinline__ float* ws_zX(const Args& a, int chain, int x)
{
    return (float*)(a.ws + a.wl.zX) + ((size_t)chain * a.wl.X + x) * a.d.Fh;
}
// Operand position of feature f: MFMA step m = f/32, lane group qg = (f%16)/4,
// slot j = 4*((f/16)%2) + f%4, position m*32 + qg*8 + j.  Lane group qg of an
// accumulator tile holds rows qg*4..qg*4+3, so tiles ft = 2m and 2m+1 of H feed
// MFMA step m without any exchange between lanes.
__device__ __forceinline__ int perm_pos(int f)
{
    const int ft = f >> 4, r = f & 15;
    return (ft >> 1) * 32 + (r >> 2) * 8 + (ft & 1) * 4 + (r & 3);
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
    if (!state_ok(a)) return;  // header mismatch or faulted state: nothing is read or written
    const int chain = blockIdx.y, b = chain / a.d.Hkv, g = chain % a.d.Hkv;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int w = a.d.w, C = a.d.C, X = a.wl.X, ns = seq_tokens(a, b);
    Chain ch = chain_of(a, chain);
    const int64_t t0 = ch.tok();
    const int cnt0 = min(max(ch.cnt(), 0), C);
    const float* W = (const float*)(a.state + a.sl.W) + (size_t)g * Fh * D;
    for (int i = threadIdx.x; i < Fh * D; i += 256) Ws[i / D][i % D] = W[i];
    if (blockIdx.x == 0 && threadIdx.x == 0 && g == 0) ((int64_t*)(a.ws + a.wl.t0))[b] = t0;
    if (blockIdx.x == 0 && threadIdx.x < 16) ((uint32_t*)(a.ws + a.wl.xsync))[chain * 16 + threadIdx.x] = 0u;
    {
        // exchange slots of the split scan start empty (exchange number 0)
        const size_t nx = (size_t)2 * (D / 16) * (C + a.d.L);
        uint64_t* xe = (uint64_t*)(a.ws + a.wl.xe) + (size_t)chain * nx;
        for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nx; i += (size_t)gridDim.x * 256) xe[i] = 0ull;
    }

    for (int rr = 0; rr < RPW; ++rr) {
        const int row = (blockIdx.x * 4 + wave) * RPW + rr;
        const T* src = nullptr;
        const T* srcv = nullptr;
        T* cpk = nullptr;
        T* cpv = nullptr;
        float* phi_out = nullptr;
        uint16_t* phs_out = nullptr;
        if (row < X) {
            phi_out = ws_phiX(a, chain, row);
            phs_out = ws_phiS(a, chain, row);
            if (row < w) {
                int64_t p = t0 - w + row;
                cpk = (T*)(a.ws + a.wl.ring0_k) + ((size_t)chain * w + row) * D;
                cpv = (T*)(a.ws + a.wl.ring0_v) + ((size_t)chain * w + row) * D;
                if (p >= 0) {
                    int slot = (int)(p % w);
                    src = ch.ring_k<T>() + (size_t)slot * D;
                    srcv = ch.ring_v<T>() + (size_t)slot * D;
                }
            } else if (row - w < ns) {  // rows past this sequence's tokens stay zero
                src = (const T*)a.k + (((size_t)b * a.n + (row - w)) * a.d.Hkv + g) * D;
            }
        } else if (row < X + C) {
            int i = row - X;
            phi_out = ws_cphi(a, chain, i);
            phs_out = ws_cphiS(a, chain, i);
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
            const bool valid = src != nullptr;
            const float p0 = valid ? ep / sp : 0.f, p1 = valid ? en / sn : 0.f;
            phi_out[lane] = p0;
            phi_out[Fh + lane] = p1;
            const uint16_t h0 = from_f32<bf16>(p0).x, h1 = from_f32<bf16>(p1).x;
            const int q0 = perm_pos(lane), q1 = perm_pos(Fh + lane);
            phs_out[q0] = h0;
            phs_out[q1] = h1;
            phs_out[2 * Fh + q0] = from_f32<bf16>(p0 - __uint_as_float((uint32_t)h0 << 16)).x;
            phs_out[2 * Fh + q1] = from_f32<bf16>(p1 - __uint_as_float((uint32_t)h1 << 16)).x;
        }
    }
}

// bf16 bits of x, rounded to nearest even (finite x), and the float a bf16 holds
__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float bf16_val(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

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

// Prologue for bf16 io: same rows and layouts, computed 16 rows per wave with
// MFMA.  z^T = W x^T uses W in three bf16 parts (the products with the bf16 key
// are exact, sums in fp32); lane (r16, qg) then holds features ft*16 + 4qg + i of
// row r16 and the two softmaxes combine the four lanes of a row by shuffles.
// grid (ceil((X + C) / 64), B*Hkv), block 256.
template <int D, int Fh>
__global__ __launch_bounds__(256) void prologue_bf16_kernel(Args a, int fp32_rows)
{
    constexpr int F = 2 * Fh, FTH = Fh / 16, DS = D / 32;
    if (!state_ok(a)) return;  // header mismatch or faulted state: nothing is read or written
    const int chain = blockIdx.y, b = chain / a.d.Hkv, g = chain % a.d.Hkv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, qg = lane >> 4;
    const int w = a.d.w, C = a.d.C, X = a.wl.X, Cp = C > 0 ? C : 1, ns = seq_tokens(a, b);
    Chain ch = chain_of(a, chain);
    const int64_t t0 = ch.tok();
    const int cnt0 = min(max(ch.cnt(), 0), C);
    // W (three bf16 parts) goes to LDS once per workgroup, every load issued before
    // any is waited for; the four waves then read their MFMA operands from there
    constexpr int WP = D + 8, WN = 3 * Fh * D / 8 / 256;  // padded row, 16-byte pieces per thread
    static_assert(3 * Fh * D % (8 * 256) == 0, "W pieces cover the workgroup exactly");
    __shared__ __attribute__((aligned(16))) uint16_t Wl[3 * Fh * WP];
    const uint16_t* Wb = (const uint16_t*)(a.state + a.sl.Wb) + (size_t)(3 * g) * Fh * D;
    {
        uint4 w4[WN];
#pragma unroll
        for (int k = 0; k < WN; ++k) w4[k] = *(const uint4*)(Wb + (size_t)(tid + k * 256) * 8);
#pragma unroll
        for (int k = 0; k < WN; ++k) {
            const int e = (tid + k * 256) * 8;  // row = part * Fh + feature
            *(uint4*)(Wl + (e / D) * WP + e % D) = w4[k];
        }
    }
    if (blockIdx.x == 0 && tid == 0 && g == 0) ((int64_t*)(a.ws + a.wl.t0))[b] = t0;
    if (blockIdx.x == 0 && tid < 16) ((uint32_t*)(a.ws + a.wl.xsync))[chain * 16 + tid] = 0u;
    {
        // exchange slots of the split scan start empty (exchange number 0)
        const size_t nx = (size_t)2 * (D / 16) * (C + a.d.L);
        uint64_t* xe = (uint64_t*)(a.ws + a.wl.xe) + (size_t)chain * nx;
        for (size_t i = (size_t)blockIdx.x * 256 + tid; i < nx; i += (size_t)gridDim.x * 256) xe[i] = 0ull;
    }
    // source key row of an extended-sequence or cache row (nullptr: none, phi = 0)
    auto row_src = [&](int row, bool v) -> const bf16* {
        if (row < w) {
            const int64_t p = t0 - w + row;
            if (p < 0) return nullptr;
            return (v ? ch.ring_v<bf16>() : ch.ring_k<bf16>()) + (size_t)(p % w) * D;
        }
        if (row < X)  // rows past this sequence's tokens: none
            return row - w < ns ? (const bf16*)(v ? a.v : a.k) + (((size_t)b * a.n + (row - w)) * a.d.Hkv + g) * D
                                : nullptr;
        if (row < X + C && row - X < cnt0) return (v ? ch.cache_v<bf16>() : ch.cache_k<bf16>()) + (size_t)(row - X) * D;
        return nullptr;
    };
    // raw copies of the window ring and the cache as they stand at the call start
    for (int idx = tid; idx < 64 * (D / 8); idx += 256) {
        const int row = blockIdx.x * 64 + idx / (D / 8), u8 = (idx % (D / 8)) * 8;
        bf16* dk = nullptr;
        bf16* dv = nullptr;
        if (row < w) {
            dk = (bf16*)(a.ws + a.wl.ring0_k) + ((size_t)chain * w + row) * D;
            dv = (bf16*)(a.ws + a.wl.ring0_v) + ((size_t)chain * w + row) * D;
        } else if (row >= X && row < X + C) {
            dk = (bf16*)(a.ws + a.wl.cache0_k) + ((size_t)chain * Cp + (row - X)) * D;
            dv = (bf16*)(a.ws + a.wl.cache0_v) + ((size_t)chain * Cp + (row - X)) * D;
        }
        if (!dk) continue;
        const bf16* sk = row_src(row, false);
        const bf16* sv = row_src(row, true);
        *(uint4*)(dk + u8) = sk ? *(const uint4*)(sk + u8) : make_uint4(0, 0, 0, 0);
        *(uint4*)(dv + u8) = sv ? *(const uint4*)(sv + u8) : make_uint4(0, 0, 0, 0);
    }
    // phi rows: this wave's 16 rows, row r16 of the tile is MFMA column r16
    const int row = blockIdx.x * 64 + wave * 16 + r16;
    const bf16* src = row < X + C ? row_src(row, false) : nullptr;
    bf16x8 xb[DS];
#pragma unroll
    for (int ks = 0; ks < DS; ++ks)
        xb[ks] = __builtin_bit_cast(bf16x8, src ? *(const uint4*)(src + ks * 32 + qg * 8) : make_uint4(0, 0, 0, 0));
    __syncthreads();  // W in LDS
    floatx4 zt[FTH];
#pragma unroll
    for (int ft = 0; ft < FTH; ++ft) {
        zt[ft] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DS; ++ks)
#pragma unroll
            for (int part = 0; part < 3; ++part)
                zt[ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    *(const bf16x8*)(Wl + (part * Fh + ft * 16 + r16) * WP + ks * 32 + qg * 8), xb[ks], zt[ft], 0, 0, 0);
    }
    float zmax = -INFINITY, zmin = INFINITY;
#pragma unroll
    for (int ft = 0; ft < FTH; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            zmax = fmaxf(zmax, zt[ft][i]);
            zmin = fminf(zmin, zt[ft][i]);
        }
    zmax = quad_max(zmax);
    zmin = quad_min(zmin);
    float ep[FTH][4], en[FTH][4], sp = 0.f, sn = 0.f;
#pragma unroll
    for (int ft = 0; ft < FTH; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ep[ft][i] = exp_acc(zt[ft][i] - zmax);
            en[ft][i] = exp_acc(zmin - zt[ft][i]);
            sp += ep[ft][i];
            sn += en[ft][i];
        }
    sp = quad_sum(sp);
    sn = quad_sum(sn);
    if (row >= X + C) return;
    if (row < X) {  // z of the row (features ft * 16 + 4 qg + i), for the state's cache_z
        float* zo = ws_zX(a, chain, row);
#pragma unroll
        for (int ft = 0; ft < FTH; ++ft) *(float4*)(zo + ft * 16 + qg * 4) = make_float4(zt[ft][0], zt[ft][1], zt[ft][2], zt[ft][3]);
    }
    const bool valid = src != nullptr;
    const float isp = valid ? 1.f / sp : 0.f, isn = valid ? 1.f / sn : 0.f;
    float ph[2 * FTH][4];  // feature tile T: + half T < FTH, - half T >= FTH
#pragma unroll
    for (int ft = 0; ft < FTH; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ph[ft][i] = ep[ft][i] * isp;
            ph[FTH + ft][i] = en[ft][i] * isn;
        }
    uint16_t* ps = row < X ? ws_phiS(a, chain, row) : ws_cphiS(a, chain, row - X);
    if (fp32_rows) {  // fp32 rows: only the one-workgroup scan reads them
        float* po = row < X ? ws_phiX(a, chain, row) : ws_cphi(a, chain, row - X);
#pragma unroll
        for (int T = 0; T < 2 * FTH; ++T)
            *(float4*)(po + T * 16 + qg * 4) = make_float4(ph[T][0], ph[T][1], ph[T][2], ph[T][3]);
    }
    // hi / lo parts in operand order: tiles 2m and 2m+1 fill positions m*32 + qg*8 + 0..7
#pragma unroll
    for (int m = 0; m < FTH; ++m) {
        u16x8 hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = ph[2 * m + (j >> 2)][j & 3];
            hi[j] = bf16_bits(x);
            lo[j] = bf16_bits(x - bf16_val(hi[j]));
        }
        *(u16x8*)(ps + m * 32 + qg * 8) = hi;
        *(u16x8*)(ps + F + m * 32 + qg * 8) = lo;
    }
}

// ---------------------------------------------------------------------------
// 2. scan: one workgroup per chain (D/16 waves), intervals in order.
//
//   Wave w owns columns [16w, 16w+16) of H: its F/16 accumulator tiles of
//   H[f][d] stay in registers across the whole call.  The same registers,
//   split into bf16 hi/lo parts, are the A operand of the SRE contraction
//   n^T = H^T phi^T for those columns, computed with three bf16 MFMAs
//   (hi.hi + lo.hi + hi.lo; each product accurate to about 2^-16 of its
//   terms, far inside the selection margin).  Every wave sees every
//   candidate: candidate phi rows (pre-split hi/lo by the prologue) and
//   values are staged through LDS 64 candidates at a time with the next
//   batch prefetched into registers; per-wave partial errors are summed in a
//   fixed order.  d = phi . s uses hi + lo in fp32.  Top-C is an exact
//   selection on (SRE desc, position asc): a 256-bin histogram over the SRE
//   bit patterns finds the boundary bin, whose few members are ranked
//   pairwise.  The fold stages up to 32 folded pairs transposed in LDS and
//   adds phi(k) v^T with phi split in three bf16 parts (exact; bf16 io, where
//   v is exact in bf16) or with fp32 MFMA (fp32 io).
// ---------------------------------------------------------------------------
constexpr int kSelBins = 256;
constexpr int kBatch = 64;      // candidates staged per SRE batch
constexpr int kFoldChunk = 64;  // folded pairs staged per fold chunk

__host__ __device__ constexpr int scan_threads(int D) { return 4 * D; }  // D/16 waves

struct ScanSmem {
    size_t stage, part, ebits, keep, fold, memb, freed, keptE, cref, cpos, hist, s, dS, ucode, bcnt, cscore, qx, red,
        misc, total;
    int sphi_stride, sv_stride;  // elements per staged phi row (bf16) / value row
};

__host__ __device__ inline ScanSmem scan_smem(int D, int F, int C, int L, int esize)
{
    ScanSmem m;
    const int U = C + L, Cp = C > 0 ? C : 1, NW = D / 16;
    m.sphi_stride = 2 * F + 8;
    m.sv_stride = D + (esize == 2 ? 8 : 4);
    const size_t sre_stage = (size_t)kBatch * (2 * m.sphi_stride + esize * m.sv_stride);
    const size_t EP = kFoldChunk + 8;
    const size_t fold_stage = esize == 2 ? 2 * EP * (3 * (size_t)F + D) : 4 * (kFoldChunk + 4) * ((size_t)F + D);
    size_t off = 0;
    m.stage = off; off += align_up(sre_stage > fold_stage ? sre_stage : fold_stage, 16);
    m.part = off;  off += sizeof(float) * (size_t)NW * U;
    m.ebits = off; off += sizeof(uint32_t) * U;
    m.keep = off;  off += sizeof(int) * U;
    m.fold = off;  off += sizeof(int) * U;
    m.memb = off;  off += sizeof(int) * U;
    m.freed = off; off += sizeof(int) * Cp;
    m.keptE = off; off += sizeof(int) * (L + 1);
    m.cref = off;  off += sizeof(int) * Cp;
    m.cpos = off;  off += sizeof(int) * Cp;
    m.hist = off;  off += sizeof(int) * kSelBins;
    m.s = off;     off += sizeof(float) * F;
    m.dS = off;    off += sizeof(float) * kBatch;
    m.ucode = off; off += sizeof(int) * U;
    m.bcnt = off;  off += sizeof(int) * 4 * ((U + 63) / 64);
    m.cscore = off; off += sizeof(float) * Cp;         // score each cached pair was kept with
    m.qx = off;    off += sizeof(float) * ((size_t)D + F);  // a query row and its features (query-based scorers)
    m.red = off;   off += sizeof(float) * 2 * 16;       // per-wave partials of block reductions
    m.misc = off;  off += sizeof(int) * 16;
    m.total = align_up(off, 16);
    return m;
}


__device__ __forceinline__ void load4(const float* p, float* o)
{
    const float4 t = *(const float4*)p;
    o[0] = t.x; o[1] = t.y; o[2] = t.z; o[3] = t.w;
}
__device__ __forceinline__ void load4(const bf16* p, float* o)
{
    const uint2 t = *(const uint2*)p;
    o[0] = __uint_as_float(t.x << 16);
    o[1] = __uint_as_float(t.x & 0xffff0000u);
    o[2] = __uint_as_float(t.y << 16);
    o[3] = __uint_as_float(t.y & 0xffff0000u);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

template <int D, int F, typename T>
__global__ __launch_bounds__(scan_threads(D)) void scan_kernel(Args a)
{
    constexpr int NT = scan_threads(D), NW = D / 16, FT = F / 16, FM = F / 32;
    constexpr int NB = kSelBins, BATCH = kBatch, EC = kFoldChunk;
    constexpr bool BF = sizeof(T) == 2;
    constexpr int VU = BF ? 8 : 4;                  // values per 16-byte unit
    constexpr int PU_ROW = (2 * F) / 8;              // 16-byte units per phi split row
    constexpr int VU_ROW = D / VU;                   // 16-byte units per value row
    constexpr int PU_PT = (BATCH * PU_ROW + NT - 1) / NT;
    constexpr int VU_PT = (BATCH * VU_ROW + NT - 1) / NT;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const Dims& d = a.d;
    const int w = d.w, C = d.C, L = d.L;
    if (!state_ok(a)) return;  // header mismatch or faulted state: nothing is read or written
    const ScanSmem sm = scan_smem(D, F, C, L, sizeof(T));
    const int SPS = sm.sphi_stride, SVS = sm.sv_stride;
    uint16_t* stP = (uint16_t*)(smem + sm.stage);                   // [BATCH][SPS]
    T* stV = (T*)(smem + sm.stage + sizeof(uint16_t) * BATCH * SPS);  // [BATCH][SVS]
    float* part = (float*)(smem + sm.part);
    uint32_t* ebits = (uint32_t*)(smem + sm.ebits);
    int* keep = (int*)(smem + sm.keep);
    int* fold = (int*)(smem + sm.fold);
    int* memb = (int*)(smem + sm.memb);
    int* freed = (int*)(smem + sm.freed);
    int* keptE = (int*)(smem + sm.keptE);
    int* cref = (int*)(smem + sm.cref);
    int* cpos = (int*)(smem + sm.cpos);
    int* hist = (int*)(smem + sm.hist);
    float* sP = (float*)(smem + sm.s);  // s in operand (perm_pos) order
    float* dS = (float*)(smem + sm.dS);
    int* ucode = (int*)(smem + sm.ucode);  // candidate source: X row (>= 0) or call-start cache slot -code-1
    int* bcnt = (int*)(smem + sm.bcnt);
    float* cscoreL = (float*)(smem + sm.cscore);
    float* qxL = (float*)(smem + sm.qx);
    float* red = (float*)(smem + sm.red);
    int* misc = (int*)(smem + sm.misc);

    const int chain = blockIdx.x, b = chain / d.Hkv, g = chain % d.Hkv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, qg = lane >> 4;
    Chain ch = chain_of(a, chain);
    const int64_t t0 = ws_t0(a, b);
    const int n = a.n, NI = a.NI;  // rows per sequence in k, v; snapshot slots per chain
    const int ns = seq_tokens(a, b), NIs = (ns + L - 1) / L;  // this sequence's tokens and intervals
    const int Cp = C > 0 ? C : 1;
    const int U = C + L;

    // ---- state in: this wave's column tiles of H to registers ----
    floatx4 Hr[FT];  // Hr[ft][i] = H[ft*16 + qg*4 + i][wave*16 + r16]
    const float* Hst = ch.H();  // [D][F]
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
        const float4 t4 = *(const float4*)(Hst + (size_t)(wave * 16 + r16) * F + ft * 16 + qg * 4);
        Hr[ft] = floatx4{t4.x, t4.y, t4.z, t4.w};
    }
    bf16x8 Ah[FM], Al[FM];  // SRE A operand: row d = wave*16 + r16, slot (qg, j) <-> feature of perm_pos
    auto split_H = [&]() {
#pragma unroll
        for (int m = 0; m < FM; ++m) {
            u16x8 h, l;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = Hr[2 * m + (j >> 2)][j & 3];
                const uint16_t hb = bf16_bits(x);
                h[j] = hb;
                l[j] = bf16_bits(x - bf16_val(hb));
            }
            Ah[m] = __builtin_bit_cast(bf16x8, h);
            Al[m] = __builtin_bit_cast(bf16x8, l);
        }
    };
    split_H();
    for (int i = tid; i < F; i += NT) sP[perm_pos(i)] = ch.s()[i];
    int cnt = min(max(ch.cnt(), 0), C);
    for (int i = tid; i < cnt; i += NT) {
        cpos[i] = ch.cpos()[i];
        cref[i] = -(i + 1);
        cscoreL[i] = ch.cscore()[i];
    }
    __syncthreads();

    float* snapH = (float*)(a.ws + a.wl.snapH) + (size_t)chain * NI * F * D;
    float* snapS = (float*)(a.ws + a.wl.snapS) + (size_t)chain * NI * F;
    int* snapRef = (int*)(a.ws + a.wl.snapRef) + (size_t)chain * NI * Cp;
    int* snapN = (int*)(a.ws + a.wl.snapN) + (size_t)chain * NI;

    for (int c = 0; c < NIs; ++c) {
        const int64_t ap = t0 + (int64_t)c * L;
        const int64_t ep = ap + L < t0 + ns ? ap + L : t0 + ns;

        // ---- interval-start snapshot (H^T [D][F], s, cache refs) ----
        {
            if constexpr (BF) {
                // the hi parts are exactly the SRE operand: features in operand order
                uint16_t* dst = (uint16_t*)(a.ws + a.wl.snapH) + ((size_t)chain * NI + c) * F * D +
                                (size_t)(wave * 16 + r16) * F + qg * 8;
#pragma unroll
                for (int m = 0; m < FM; ++m) *(bf16x8*)(dst + m * 32) = Ah[m];
            } else {
                float* dst = snapH + (size_t)c * F * D + (size_t)(wave * 16 + r16) * F + qg * 4;
#pragma unroll
                for (int ft = 0; ft < FT; ++ft)
                    *(float4*)(dst + ft * 16) = make_float4(Hr[ft][0], Hr[ft][1], Hr[ft][2], Hr[ft][3]);
            }
            for (int i = tid; i < F; i += NT) snapS[(size_t)c * F + i] = sP[perm_pos(i)];
            for (int i = tid; i < cnt; i += NT) snapRef[(size_t)c * Cp + i] = cref[i];
            if (tid == 0) snapN[c] = cnt;
        }

        // ---- candidates: cache slots [0, cnt) then the keys leaving the window ----
        const int64_t eS = ap - w > 0 ? ap - w : 0;
        const int64_t eE = ep - w;
        const int nE = eE > eS ? (int)(eE - eS) : 0;
        const int nU = cnt + nE;
        const int xE0 = (int)(eS - (t0 - w));
        for (int u = tid; u < nU; u += NT) ucode[u] = u < cnt ? cref[u] : xE0 + (u - cnt);
        const float* phiX0 = ws_phiX(a, chain, 0);
        const float* cphi0 = ws_cphi(a, chain, 0);
        const uint16_t* phiS0 = ws_phiS(a, chain, 0);
        const uint16_t* cphiS0 = ws_cphiS(a, chain, 0);
        const T* vin0 = (const T*)a.v + ((size_t)b * n * d.Hkv + g) * D;   // + (x - w) * Hkv * D
        const T* ring0v = (const T*)(a.ws + a.wl.ring0_v) + (size_t)chain * w * D;
        const T* cache0v = (const T*)(a.ws + a.wl.cache0_v) + (size_t)chain * Cp * D;
        auto code_phi = [&](int code) -> const float* {
            return code >= 0 ? phiX0 + (size_t)code * F : cphi0 + (size_t)(-code - 1) * F;
        };
        auto code_phs = [&](int code) -> const uint16_t* {
            return code >= 0 ? phiS0 + (size_t)code * 2 * F : cphiS0 + (size_t)(-code - 1) * 2 * F;
        };
        auto code_v = [&](int code) -> const T* {
            const T* pin = vin0 + (size_t)(code - w) * d.Hkv * D;
            const T* pring = ring0v + (size_t)code * D;
            const T* pcache = cache0v + (size_t)(-code - 1) * D;
            return code >= w ? pin : (code >= 0 ? pring : pcache);
        };
        auto cand_phi = [&](int u) -> const float* { return code_phi(ucode[u]); };
        auto cand_v = [&](int u) -> const T* { return code_v(ucode[u]); };
        auto cand_pos = [&](int u) -> int { return u < cnt ? cpos[u] : (int)(eS + (u - cnt)); };
        // Block-wide max or sum of one value per thread (every thread gets the result).
        auto block_op = [&](float x, bool is_max) -> float {
            x = is_max ? wave_max(x) : wave_sum(x);
            __syncthreads();  // the previous result has been read
            if (lane == 0) red[wave] = x;
            __syncthreads();
            float r = red[0];
            for (int ww = 1; ww < NW; ++ww) r = is_max ? fmaxf(r, red[ww]) : r + red[ww];
            return r;
        };
        // Scores of the policies other than the SRE (lola_policy in lola.h): the stored
        // score of each cached pair; or, head by head, the interval's last query against
        // every candidate: its softmax weight among the candidates (fp32 logits, expf)
        // and, for the approximation error, the candidate's normalised feature weight.
        float* score = part;  // candidate u's score, once the SRE partials are summed
        auto policy_scores = [&](int nUq, int64_t epq) {
            const int pol = d.policy;
            if (pol == LOLA_POLICY_SRE_STALE) {
                for (int u = tid; u < cnt; u += NT) score[u] = cscoreL[u];
                return;
            }
            if (pol != LOLA_POLICY_ATTN && pol != LOLA_POLICY_SOFTMAX_ERR) return;
            float* lgt = part + U;      // (the partial-SRE rows of waves 1 and 2 are free now)
            float* kap = part + 2 * U;
            float* qv = qxL;
            float* phq = qxL + D;
            const int G = d.G;
            const size_t trow = (size_t)(epq - 1 - t0);  // row of the interval's last query in this call
            for (int u = tid; u < nUq; u += NT) score[u] = 0.f;
            for (int h = 0; h < G; ++h) {
                __syncthreads();  // the previous head's rows are consumed
                const T* qp = (const T*)a.q + (((size_t)b * n + trow) * d.Hq + (size_t)g * G + h) * D;
                for (int i = tid; i < D; i += NT) qv[i] = to_f32(qp[i]);
                __syncthreads();
                if (pol == LOLA_POLICY_SOFTMAX_ERR) {
                    if (wave == 0) {  // phi(q) = [softmax(W q); softmax(-W q)], lane i < F/2 holds (W q)_i
                        const float* Wg = (const float*)(a.state + a.sl.W) + (size_t)g * (F / 2) * D;
                        float z = 0.f;
                        if (lane < F / 2)
                            for (int j = 0; j < D; ++j) z += Wg[(size_t)lane * D + j] * qv[j];
                        const float zmax = wave_max(lane < F / 2 ? z : -INFINITY);
                        const float zmin = -wave_max(lane < F / 2 ? -z : -INFINITY);
                        const float e1 = lane < F / 2 ? expf(z - zmax) : 0.f;
                        const float e2 = lane < F / 2 ? expf(zmin - z) : 0.f;
                        const float s1 = wave_sum(e1), s2 = wave_sum(e2);
                        if (lane < F / 2) {
                            phq[lane] = e1 / s1;
                            phq[F / 2 + lane] = e2 / s2;
                        }
                    }
                    __syncthreads();
                }
                float mx = -INFINITY, ks = 0.f;
                for (int u = tid; u < nUq; u += NT) {
                    const int code = ucode[u];
                    const T* kr = ref_k<T>(a, chain, b, g, code);
                    float dot = 0.f;
                    for (int j = 0; j < D; j += 4) {
                        float x[4];
                        load4(kr + j, x);
                        dot += qv[j] * x[0] + qv[j + 1] * x[1] + qv[j + 2] * x[2] + qv[j + 3] * x[3];
                    }
                    const float l = d.tau * dot;
                    lgt[u] = l;
                    mx = fmaxf(mx, l);
                    if (pol == LOLA_POLICY_SOFTMAX_ERR) {
                        const float* pr = code_phi(code);
                        float kk = 0.f;
                        for (int f = 0; f < F; f += 4) {
                            float x[4];
                            load4(pr + f, x);
                            kk += phq[f] * x[0] + phq[f + 1] * x[1] + phq[f + 2] * x[2] + phq[f + 3] * x[3];
                        }
                        kap[u] = kk;
                        ks += kk;
                    }
                }
                mx = block_op(mx, true);
                if (pol == LOLA_POLICY_SOFTMAX_ERR) ks = block_op(ks, false);
                float zs = 0.f;
                for (int u = tid; u < nUq; u += NT) zs += expf(lgt[u] - mx);
                zs = block_op(zs, false);
                for (int u = tid; u < nUq; u += NT) {
                    const float p = expf(lgt[u] - mx) / zs;
                    score[u] += pol == LOLA_POLICY_ATTN ? p : fabsf(p - kap[u] / ks);
                }
            }
        };
        __syncthreads();  // codes ready

        // ---- SRE in batches of 64 candidates ----
        const int nbat = (nU + BATCH - 1) / BATCH;
        uint4 pre_p[PU_PT], pre_v[VU_PT];
        auto prefetch = [&](int bi) {
#pragma unroll
            for (int k = 0; k < PU_PT; ++k) {
                const int idx = tid + k * NT;
                const int cl = idx / PU_ROW, un = idx % PU_ROW, u = bi * BATCH + cl;
                const bool ok = idx < BATCH * PU_ROW && u < nU;
                const uint4 t4 = *(const uint4*)(code_phs(ucode[ok ? u : 0]) + un * 8);
                pre_p[k] = ok ? t4 : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int k = 0; k < VU_PT; ++k) {
                const int idx = tid + k * NT;
                const int cl = idx / VU_ROW, un = idx % VU_ROW, u = bi * BATCH + cl;
                const bool ok = idx < BATCH * VU_ROW && u < nU;
                const uint4 t4 = *(const uint4*)(code_v(ucode[ok ? u : 0]) + un * VU);
                pre_v[k] = ok ? t4 : make_uint4(0, 0, 0, 0);
            }
        };
        if (nbat > 0) prefetch(0);
        for (int bi = 0; bi < nbat; ++bi) {
            __syncthreads();  // the previous batch is consumed
#pragma unroll
            for (int k = 0; k < PU_PT; ++k) {
                const int idx = tid + k * NT;
                if (idx < BATCH * PU_ROW) *(uint4*)(stP + (idx / PU_ROW) * SPS + (idx % PU_ROW) * 8) = pre_p[k];
            }
#pragma unroll
            for (int k = 0; k < VU_PT; ++k) {
                const int idx = tid + k * NT;
                if (idx < BATCH * VU_ROW) *(uint4*)(stV + (idx / VU_ROW) * SVS + (idx % VU_ROW) * VU) = pre_v[k];
            }
            __syncthreads();
            if (bi + 1 < nbat) prefetch(bi + 1);
            {
                // d = phi . s for the staged candidates, (hi + lo) parts in fp32;
                // wave w takes BATCH/NW candidates, LPC lanes per candidate
                constexpr int CPW = BATCH / NW, LPC = 64 / CPW, PPL = F / LPC;
                const int cl = wave * CPW + lane / LPC, sub = lane % LPC;
                const uint16_t* pr = stP + cl * SPS + sub * PPL;
                float dd = 0.f;
#pragma unroll
                for (int p = 0; p < PPL; p += 8) {
                    const uint4 hq = *(const uint4*)(pr + p);
                    const uint4 lq = *(const uint4*)(pr + F + p);
                    const float4 s0 = *(const float4*)(sP + sub * PPL + p);
                    const float4 s1 = *(const float4*)(sP + sub * PPL + p + 4);
                    const uint32_t hw[4] = {hq.x, hq.y, hq.z, hq.w}, lw[4] = {lq.x, lq.y, lq.z, lq.w};
                    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float hv = __uint_as_float((j & 1) ? (hw[j >> 1] & 0xffff0000u) : (hw[j >> 1] << 16));
                        const float lv = __uint_as_float((j & 1) ? (lw[j >> 1] & 0xffff0000u) : (lw[j >> 1] << 16));
                        dd += (hv + lv) * sv[j];
                    }
                }
#pragma unroll
                for (int o = 1; o < LPC; o <<= 1) dd += __shfl_xor(dd, o, 64);
                if (sub == 0) dS[cl] = dd;
            }
            __syncthreads();
#pragma unroll
            for (int tl = 0; tl < BATCH / 16; tl += 2) {
                if (bi * BATCH + tl * 16 >= nU) break;  // wave-uniform; rows past nU are zero-filled
                floatx4 acc[2], acc2[2];
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2) acc[t2] = acc2[t2] = floatx4{0.f, 0.f, 0.f, 0.f};
                const uint16_t* pr0 = stP + (tl * 16 + r16) * SPS + qg * 8;
                const uint16_t* pr1 = pr0 + 16 * SPS;
#pragma unroll
                for (int m = 0; m < FM; ++m) {
                    const bf16x8 h0 = *(const bf16x8*)(pr0 + m * 32);
                    const bf16x8 h1 = *(const bf16x8*)(pr1 + m * 32);
                    const bf16x8 l0 = *(const bf16x8*)(pr0 + F + m * 32);
                    const bf16x8 l1 = *(const bf16x8*)(pr1 + F + m * 32);
                    acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah[m], h0, acc[0], 0, 0, 0);
                    acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah[m], h1, acc[1], 0, 0, 0);
                    acc2[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al[m], h0, acc2[0], 0, 0, 0);
                    acc2[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al[m], h1, acc2[1], 0, 0, 0);
                    acc2[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah[m], l0, acc2[0], 0, 0, 0);
                    acc2[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah[m], l1, acc2[1], 0, 0, 0);
                }
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2) {
                    const int cl = (tl + t2) * 16 + r16;
                    const int u = bi * BATCH + cl;
                    const float dpart = dS[cl];
                    const float inv = dpart > 0.f ? 1.0f / dpart : 0.f;
                    // n[d = wave*16 + qg*4 + i][candidate u] = acc + acc2
                    float vv[4];
                    load4(stV + cl * SVS + wave * 16 + qg * 4, vv);
                    float e = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float df = (acc[t2][i] + acc2[t2][i]) * inv - vv[i];
                        e += df * df;
                    }
                    e = quad_sum(e);
                    if (qg == 0 && u < nU) part[wave * U + u] = e;
                }
            }
        }
        __syncthreads();  // per-wave partial errors complete

        // ---- scores: the SRE totals (part[u] once summed), or the policy's score ----
        for (int u = tid; u < nU; u += NT) {
            float e = part[u];
#pragma unroll
            for (int ww = 1; ww < NW; ++ww) e += part[ww * U + u];
            score[u] = e;
        }
        if (d.policy != LOLA_POLICY_SRE && nU > 0) {  // block-uniform
            __syncthreads();
            policy_scores(nU, ep);
        }
        // ---- exact top-C on (score desc, position asc), all waves ----
        {
            uint32_t lo = 0xffffffffu, hi = 0u;
            for (int u = tid; u < nU; u += NT) {
                // scores are >= 0, so their bit patterns order like them; FIFO orders by position
                const uint32_t eb = d.policy == LOLA_POLICY_FIFO ? (uint32_t)cand_pos(u) : __float_as_uint(score[u]);
                ebits[u] = eb;
                lo = min(lo, eb);
                hi = max(hi, eb);
            }
            lo = wave_min_u32(lo);
            hi = wave_max_u32(hi);
            if (tid == 0) { misc[0] = (int)lo; misc[1] = (int)hi; misc[2] = 0; }
            for (int i = tid; i < NB; i += NT) hist[i] = 0;
            __syncthreads();
            if (lane == 0 && wave > 0) { atomicMin((uint32_t*)&misc[0], lo); atomicMax((uint32_t*)&misc[1], hi); }
        }
        __syncthreads();
        if (nU > C && C > 0) {
            const uint32_t minb = (uint32_t)misc[0];
            // monotone bin of an SRE bit pattern (same formula in every pass)
            const float bscale = (float)NB / ((float)((uint32_t)misc[1] - minb) + 1.0f);
            auto bin_of = [&](uint32_t x) { return min(NB - 1, (int)((float)(x - minb) * bscale)); };
            for (int u = tid; u < nU; u += NT) atomicAdd(&hist[bin_of(ebits[u])], 1);
            __syncthreads();
            // every wave scans the bins (highest first; lane l holds bins NB-1-4l .. NB-4-4l)
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
            const int m = misc[2];
            for (int i = tid; i < m; i += NT) {
                const int u = memb[i];
                const uint32_t eu = ebits[u];
                const int pu = cand_pos(u);
                int rank = 0;
                for (int j2 = 0; j2 < m; ++j2) {
                    const int v2 = memb[j2];
                    const uint32_t ev = ebits[v2];
                    rank += (ev > eu) || (ev == eu && cand_pos(v2) < pu);
                }
                keep[u] = rank < need;
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

        // ---- fold: H += sum phi(k) v^T, s += sum phi(k), 32 pairs at a time ----
        for (int e0 = 0; e0 < nF; e0 += EC) {
            const int ne = nF - e0 < EC ? nF - e0 : EC;
            if (e0 > 0) __syncthreads();  // the previous chunk is consumed
            if constexpr (BF) {
                constexpr int EP = EC + 8;
                uint16_t* P1 = (uint16_t*)(smem + sm.stage);  // [3][F][EP]
                uint16_t* VTb = P1 + 3 * F * EP;             // [D][EP]
                for (int idx = tid; idx < EC * (F / 4); idx += NT) {
                    const int e1 = idx % EC, f4 = (idx / EC) * 4;
                    float x[4] = {0.f, 0.f, 0.f, 0.f};
                    if (e1 < ne) load4(cand_phi(fold[e0 + e1]) + f4, x);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint16_t p1 = bf16_bits(x[k]);
                        const float r1 = x[k] - bf16_val(p1);
                        const uint16_t p2 = bf16_bits(r1);
                        const uint16_t p3 = bf16_bits(r1 - bf16_val(p2));
                        P1[(f4 + k) * EP + e1] = p1;
                        P1[F * EP + (f4 + k) * EP + e1] = p2;
                        P1[2 * F * EP + (f4 + k) * EP + e1] = p3;
                    }
                }
                for (int idx = tid; idx < EC * (D / 8); idx += NT) {
                    const int e1 = idx % EC, d8 = (idx / EC) * 8;
                    uint4 t4 = make_uint4(0, 0, 0, 0);
                    if (e1 < ne) t4 = *(const uint4*)(cand_v(fold[e0 + e1]) + d8);
                    const uint32_t tw[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
                    for (int k = 0; k < 8; ++k) VTb[(d8 + k) * EP + e1] = (uint16_t)(tw[k >> 1] >> (16 * (k & 1)));
                }
                __syncthreads();
                // s += phi^T 1: one feature tile per wave, B operand of ones (exact)
                {
                    const bf16x8 ones = __builtin_bit_cast(bf16x8, u16x8{0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80});
                    for (int ft = wave; ft < FT; ft += NW) {
                        floatx4 sa = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < EC / 32; ++ks) {
                            const int o = (ft * 16 + r16) * EP + ks * 32 + qg * 8;
                            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(P1 + o), ones, sa, 0, 0, 0);
                            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(P1 + F * EP + o), ones, sa, 0, 0, 0);
                            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(P1 + 2 * F * EP + o), ones, sa, 0, 0, 0);
                        }
                        if (r16 == 0)
#pragma unroll
                            for (int i = 0; i < 4; ++i) sP[perm_pos(ft * 16 + qg * 4 + i)] += sa[i];
                    }
                }
#pragma unroll
                for (int ks = 0; ks < EC / 32; ++ks) {
                    const bf16x8 bv = *(const bf16x8*)(VTb + (wave * 16 + r16) * EP + ks * 32 + qg * 8);
#pragma unroll
                    for (int ft = 0; ft < FT; ++ft) {
                        const int o = (ft * 16 + r16) * EP + ks * 32 + qg * 8;
                        Hr[ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(P1 + o), bv, Hr[ft], 0, 0, 0);
                        Hr[ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(P1 + F * EP + o), bv, Hr[ft], 0, 0, 0);
                        Hr[ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(P1 + 2 * F * EP + o), bv, Hr[ft], 0,
                                                                         0, 0);
                    }
                }
            } else {
                constexpr int EP = EC + 4;
                float* PhT = (float*)(smem + sm.stage);  // [F][EP]
                float* VTf = PhT + F * EP;               // [D][EP]
                for (int idx = tid; idx < EC * (F / 4); idx += NT) {
                    const int e1 = idx % EC, f4 = (idx / EC) * 4;
                    float x[4] = {0.f, 0.f, 0.f, 0.f};
                    if (e1 < ne) load4(cand_phi(fold[e0 + e1]) + f4, x);
#pragma unroll
                    for (int k = 0; k < 4; ++k) PhT[(f4 + k) * EP + e1] = x[k];
                }
                for (int idx = tid; idx < EC * (D / 4); idx += NT) {
                    const int e1 = idx % EC, d4 = (idx / EC) * 4;
                    float x[4] = {0.f, 0.f, 0.f, 0.f};
                    if (e1 < ne) load4(cand_v(fold[e0 + e1]) + d4, x);
#pragma unroll
                    for (int k = 0; k < 4; ++k) VTf[(d4 + k) * EP + e1] = x[k];
                }
                __syncthreads();
                for (int ft = wave; ft < FT; ft += NW) {
                    floatx4 sa = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < EC / 4; ++kk)
                        sa = __builtin_amdgcn_mfma_f32_16x16x4f32(PhT[(ft * 16 + r16) * EP + kk * 4 + qg], 1.0f, sa, 0, 0, 0);
                    if (r16 == 0)
#pragma unroll
                        for (int i = 0; i < 4; ++i) sP[perm_pos(ft * 16 + qg * 4 + i)] += sa[i];
                }
#pragma unroll
                for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                    for (int kk = 0; kk < EC / 4; ++kk)
                        Hr[ft] = __builtin_amdgcn_mfma_f32_16x16x4f32(PhT[(ft * 16 + r16) * EP + kk * 4 + qg],
                                                                      VTf[(wave * 16 + r16) * EP + kk * 4 + qg], Hr[ft],
                                                                      0, 0, 0);
            }
        }

        // ---- new bf16 parts of H; kept leaving keys take freed slots, then new slots ----
        if (nF > 0) split_H();
        for (int i = tid; i < nK; i += NT) {
            const int u = keptE[i];
            const int slot = i < nFr ? freed[i] : cnt + (i - nFr);
            cref[slot] = xE0 + (u - cnt);
            cpos[slot] = (int)(eS + (u - cnt));
            cscoreL[slot] = score[u];
        }
        cnt = nU < C ? nU : C;
        __syncthreads();
    }

    // ---- state out ----
    float* Hd = ch.H();
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
        *(float4*)(Hd + (size_t)(wave * 16 + r16) * F + ft * 16 + qg * 4) =
            make_float4(Hr[ft][0], Hr[ft][1], Hr[ft][2], Hr[ft][3]);
    for (int i = tid; i < F; i += NT) ch.s()[i] = sP[perm_pos(i)];
    for (int i = tid; i < cnt; i += NT) {
        ch.cpos()[i] = cpos[i];
        ch.cscore()[i] = cscoreL[i];
    }
    // cache and window rows in 16-byte pieces
    constexpr int EP = 16 / (int)sizeof(T), NP = D / EP;
    static_assert(D % EP == 0, "rows are whole 16-byte pieces");
    for (int q = tid; q < cnt * NP; q += NT) {
        const int i = q / NP, pc = (q % NP) * EP, code = cref[i];
        if (code >= 0) {
            const uint4 k4 = *(const uint4*)(xrow_k<T>(a, chain, b, g, code) + pc);
            const uint4 v4 = *(const uint4*)(xrow_v<T>(a, chain, b, g, code) + pc);
            *(uint4*)(ch.cache_k<T>() + (size_t)i * D + pc) = k4;
            *(uint4*)(ch.cache_v<T>() + (size_t)i * D + pc) = v4;
        }
    }
    if constexpr (std::is_same<T, bf16>::value) {
        // z = W k of the cache entries added in this call
        constexpr int ZP = F / 2 / 4;
        for (int q = tid; q < cnt * ZP; q += NT) {
            const int i = q / ZP, pc = (q % ZP) * 4, code = cref[i];
            if (code >= 0) *(float4*)(ch.cz() + (size_t)i * (F / 2) + pc) = *(const float4*)(ws_zX(a, chain, code) + pc);
        }
    }
    if (w > 0) {
        const int64_t tend = t0 + ns;
        const int64_t p0 = tend - w > t0 ? tend - w : t0;
        const int nr = (int)(tend - p0);
        for (int q = tid; q < nr * NP; q += NT) {
            const int i = q / NP, pc = (q % NP) * EP;
            const int64_t p = p0 + i;
            const int slot = (int)(p % w);
            const size_t src = (((size_t)b * n + (size_t)(p - t0)) * d.Hkv + g) * D + pc;
            *(uint4*)(ch.ring_k<T>() + (size_t)slot * D + pc) = *(const uint4*)((const T*)a.k + src);
            *(uint4*)(ch.ring_v<T>() + (size_t)slot * D + pc) = *(const uint4*)((const T*)a.v + src);
        }
    }
    if (tid == 0) {
        ch.cnt() = cnt;
        ch.tok() = t0 + ns;
        ch.incv() = 0;  // stored incremental decode scores no longer match
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
    if (!state_ok(a)) return;  // header mismatch or faulted state: nothing is read or written
    const Dims& d = a.d;
    const int G = d.G, L = d.L, w = d.w;
    const int chain = blockIdx.y, b = chain / d.Hkv, g = chain % d.Hkv;
    const int rows = G * L;
    const int wpi = (rows + 63) / 64;
    const int c = blockIdx.x / wpi, rblk = blockIdx.x % wpi;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15, qg = lane >> 4;
    const int ns = seq_tokens(a, b);
    if ((int64_t)c * L >= ns) return;  // past this sequence's tokens (the whole workgroup)
    const int64_t t0 = ws_t0(a, b);
    const int64_t ap = t0 + (int64_t)c * L;
    const int64_t ep = ap + L < t0 + ns ? ap + L : t0 + ns;
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
        zmax = quad_max(zmax);
        zmin = quad_min(zmin);
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
        sp = quad_sum(sp);
        sn = quad_sum(sn);
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
            for (int j = 0; j < KPL; ++j) tmp[j] = sH[(size_t)(dt * 16 + r16) * F + held_feature<Fh>(qg, mf * KPL + j)];
            O[dt] = M::mma(M::pack(tmp), pf[mf], O[dt]);
        }
    }
    float zl = 0.f;
#pragma unroll
    for (int j = 0; j < NH; ++j) zl += hq[j] * sS[held_feature<Fh>(qg, j)];
    zl = quad_sum(zl);
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
        bmax = quad_max(bmax);
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
    Z = quad_sum(Z);
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
