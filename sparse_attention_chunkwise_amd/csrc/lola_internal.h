// Internal definitions shared by the HIP sources of liblola: the state and
// workspace layouts, bf16 storage conversion and the MFMA operand traits.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lola.h"

namespace lola {

// ---------------------------------------------------------------------------
// sizes and limits
// ---------------------------------------------------------------------------
constexpr int kMaxGroup = 16;     // query heads per KV head
constexpr int kMaxWindow = 8192;
constexpr int kMaxCache = 1024;
constexpr int kMaxChunk = 256;
constexpr int kMaxCand = kMaxCache + kMaxChunk;  // |cache| + |leaving keys| per interval
constexpr uint32_t kMagic = 0x414c4f4cu;         // "LOLA"
constexpr uint32_t kVersion = 4;

constexpr __host__ __device__ size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Combine the four lanes l, l ^ 16, l ^ 32, l ^ 48 of a wave: op(x, x^16) first, then
// op with the same of lane ^ 32, as two __shfl_xor steps would (same operands, same
// order), but with the lane-swap instructions of gfx950 (VALU, no LDS round trip).
// Each swap leaves one of the two partners' values in each output register.
#define LOLA_QUAD_COMBINE(name, OP)                                                             \
    __device__ __forceinline__ float name(float x)                                              \
    {                                                                                           \
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), \
                                                        false, false);                          \
        x = OP(__uint_as_float(a[0]), __uint_as_float(a[1]));                                   \
        const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), \
                                                        false, false);                          \
        return OP(__uint_as_float(b[0]), __uint_as_float(b[1]));                                \
    }
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(0xc07f); }  // lgkmcnt(0)

// Block barrier that orders LDS only: global loads stay in flight across it
// (a full __syncthreads would wait for every outstanding load and store).
__device__ __forceinline__ void lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float lola_add(float a, float b) { return a + b; }
LOLA_QUAD_COMBINE(quad_sum, lola_add)
LOLA_QUAD_COMBINE(quad_max, fmaxf)
LOLA_QUAD_COMBINE(quad_min, fminf)
#undef LOLA_QUAD_COMBINE

struct Dims {
    int Hq, Hkv, D, Fh, F, w, C, L, G;
    int io;       // 0 = f32, 1 = bf16
    int esize;    // bytes per io element
    float tau;    // softmax scale on q.k
    int policy;   // lola_policy
    int inc;      // 1: the state keeps n = H^T phi(k), d = s . phi(k) per cached pair (incremental decode)
};

struct StateHeader {
    uint32_t magic;
    uint32_t version;
    uint64_t cfg_hash;
    int32_t batch;
    int32_t fault;  // nonzero once a prefill scan gave up waiting for a sibling workgroup
    int32_t pad[2];
};
static_assert(sizeof(StateHeader) == 32, "kernels test the first 32 bytes of a state");

// State buffer: header | W [Hkv][Fh][D] f32 | Wb [Hkv][3][Fh][D] bf16 (three parts of W, largest first) | chains [B][Hkv]
// chain: tokens seen i64 | cache_count i32 | H^T [D][F] f32 | s [F] f32 | cache_pos [C] i32 |
//        ring_k [w][D] io | ring_v [w][D] io | cache_k [C][D] io | cache_v [C][D] io |
//        cache_z [C][Fh] f32 (bf16 io only: z = W k of each cached key, from which a
//        decode step recomputes phi(k) = [softmax(z); softmax(-z)] without the W
//        product) | cache_score [C] f32 (the score each cached
//        pair was kept with; the stale-score policy reads it back) |
//        incremental decode only: cache_n [C][D] f32 (H^T phi(k) of each cached pair),
//        cache_d [C] f32 (s . phi(k)); the int32 at chain offset 12 is 1 while they
//        match the state (a prefill call sets it to 0)
// Every chain keeps its own token count so that concurrent chains of one
// sequence never race on a shared counter.  The window ring slot of
// position p is p % w.
struct StateLayout {
    size_t W, Wb, chains, chain_bytes;
    size_t otok, ocnt, oincv, oH, os, ocpos, oring_k, oring_v, ocache_k, ocache_v, ocz, oscore, ocn, ocd;
    size_t total;
};

inline __host__ __device__ StateLayout state_layout(const Dims& d, int B)
{
    StateLayout s;
    size_t off = 256;
    s.W = off;
    off = align_up(off + sizeof(float) * (size_t)d.Hkv * d.Fh * d.D, 256);
    s.Wb = off;
    off = align_up(off + sizeof(uint16_t) * 3 * (size_t)d.Hkv * d.Fh * d.D, 256);
    s.chains = off;
    size_t c = 0;
    s.otok = 0;
    s.ocnt = 8;
    s.oincv = 12;    c = 256;
    s.oH = c;        c = align_up(c + sizeof(float) * (size_t)d.F * d.D, 256);
    s.os = c;        c = align_up(c + sizeof(float) * (size_t)d.F, 256);
    s.ocpos = c;     c = align_up(c + sizeof(int32_t) * (size_t)(d.C > 0 ? d.C : 1), 256);
    s.oring_k = c;   c = align_up(c + (size_t)d.esize * d.w * d.D, 256);
    s.oring_v = c;   c = align_up(c + (size_t)d.esize * d.w * d.D, 256);
    s.ocache_k = c;  c = align_up(c + (size_t)d.esize * d.C * d.D, 256);
    s.ocache_v = c;  c = align_up(c + (size_t)d.esize * d.C * d.D, 256);
    s.ocz = c;       c = align_up(c + (d.io == 1 ? sizeof(float) * (size_t)d.Fh * d.C : 0), 256);
    s.oscore = c;    c = align_up(c + sizeof(float) * (size_t)(d.C > 0 ? d.C : 1), 256);
    s.ocn = c;       c = align_up(c + (d.inc ? sizeof(float) * (size_t)d.C * d.D : 0), 256);
    s.ocd = c;       c = align_up(c + (d.inc ? sizeof(float) * (size_t)d.C : 0), 256);
    s.chain_bytes = c;
    s.total = s.chains + c * (size_t)B * d.Hkv;
    return s;
}

// Prefill workspace for one call of n tokens (X = w + n rows of the extended
// sequence: the window at the call start followed by the new tokens).
//   t0 [B] i64 | phiX [B][Hkv][X][F] f32 | ring0_k/v [B][Hkv][w][D] io |
//   cache0_k/v [B][Hkv][C][D] io | cphi [B][Hkv][C][F] f32 |
//   phiS [B][Hkv][X][2F] bf16 | cphiS [B][Hkv][C][2F] bf16 (hi then lo parts of
//   phi, features in the SRE operand order) | zX [B][Hkv][X][Fh] f32 (bf16 io: z = W k
//   of each row, for the state's cache_z) |
//   snapH [B][Hkv][NI][D][F] H^T: f32 for f32 io; bf16 (hi part) in operand order for bf16 io |
//   snapS [B][Hkv][NI][F] f32 |
//   snapRef [B][Hkv][NI][C] i32 | snapN [B][Hkv][NI] i32 |
//   xsync [B][Hkv][16] u32 (give-up flag, reads-done counter) |
//   xe [B][Hkv][2][D/16][C + L] u64 (per-column-slice partial SRE: exchange
//      number << 32 | f32 bits; two buffers used alternately)
struct WsLayout {
    size_t t0, phiX, ring0_k, ring0_v, cache0_k, cache0_v, cphi, phiS, cphiS, zX, snapH, snapS, snapRef, snapN, xsync, xe;
    size_t total;
    int X, NI;
};

inline __host__ __device__ WsLayout ws_layout(const Dims& d, int B, int n)
{
    WsLayout s;
    s.X = d.w + n;
    s.NI = (n + d.L - 1) / d.L;
    size_t ch = (size_t)B * d.Hkv;
    int Cp = d.C > 0 ? d.C : 1;
    size_t off = 0;
    s.t0 = off;       off = align_up(off + sizeof(int64_t) * (size_t)B, 256);
    s.phiX = off;     off = align_up(off + sizeof(float) * ch * s.X * d.F, 256);
    s.ring0_k = off;  off = align_up(off + (size_t)d.esize * ch * d.w * d.D, 256);
    s.ring0_v = off;  off = align_up(off + (size_t)d.esize * ch * d.w * d.D, 256);
    s.cache0_k = off; off = align_up(off + (size_t)d.esize * ch * Cp * d.D, 256);
    s.cache0_v = off; off = align_up(off + (size_t)d.esize * ch * Cp * d.D, 256);
    s.cphi = off;     off = align_up(off + sizeof(float) * ch * Cp * d.F, 256);
    s.phiS = off;     off = align_up(off + sizeof(uint16_t) * ch * s.X * 2 * d.F, 256);
    s.cphiS = off;    off = align_up(off + sizeof(uint16_t) * ch * Cp * 2 * d.F, 256);
    s.zX = off;       off = align_up(off + (d.io == 1 ? sizeof(float) * ch * s.X * d.Fh : 0), 256);
    s.snapH = off;    off = align_up(off + (size_t)(d.io == 1 ? 2 : 4) * ch * s.NI * d.F * d.D, 256);
    s.snapS = off;    off = align_up(off + sizeof(float) * ch * s.NI * d.F, 256);
    s.snapRef = off;  off = align_up(off + sizeof(int32_t) * ch * s.NI * Cp, 256);
    s.snapN = off;    off = align_up(off + sizeof(int32_t) * ch * s.NI, 256);
    s.xsync = off;    off = align_up(off + sizeof(uint32_t) * 16 * ch, 256);
    s.xe = off;       off = align_up(off + sizeof(uint64_t) * ch * 2 * (d.D / 16) * (size_t)(d.C + d.L), 256);
    s.total = off;
    return s;
}

// ---------------------------------------------------------------------------
// bf16 storage (round to nearest even on store)
// ---------------------------------------------------------------------------
struct bf16 {
    uint16_t x;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return __uint_as_float((uint32_t)v.x << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v)
{
    uint32_t u = __float_as_uint(v);
    bf16 r;
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
        r.x = (uint16_t)((u >> 16) | 0x40);  // quiet NaN
    } else {
        u += 0x7fffu + ((u >> 16) & 1u);
        r.x = (uint16_t)(u >> 16);
    }
    return r;
}

// ---------------------------------------------------------------------------
// MFMA operand traits.  Both shapes produce a 16x16 f32 tile; lane l holds
// C[4*(l/16) + i][l%16], i = 0..3.  An A (B) operand lane holds KPL values of
// row (column) l%16 at contraction slots (l/16)*KPL + j.
// ---------------------------------------------------------------------------
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

template <typename T> struct Mma;

template <> struct Mma<float> {       // v_mfma_f32_16x16x4_f32: exact fp32 products
    static constexpr int KPL = 1;
    using frag = float;
    __device__ __forceinline__ static frag pack(const float* v) { return v[0]; }
    __device__ __forceinline__ static frag zero() { return 0.f; }
    __device__ __forceinline__ static floatx4 mma(frag a, frag b, floatx4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<bf16> {        // v_mfma_f32_16x16x32_bf16 (gfx950)
    static constexpr int KPL = 8;
    using frag = bf16x8;
    __device__ __forceinline__ static frag pack(const float* v)
    {
        u16x8 u;
#pragma unroll
        for (int j = 0; j < 8; ++j) u[j] = from_f32<bf16>(v[j]).x;
        return __builtin_bit_cast(bf16x8, u);
    }
    __device__ __forceinline__ static frag zero() { return __builtin_bit_cast(bf16x8, u16x8{0, 0, 0, 0, 0, 0, 0, 0}); }
    __device__ __forceinline__ static floatx4 mma(frag a, frag b, floatx4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

// ---------------------------------------------------------------------------
// wave helpers (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Kernel argument bundle common to the launches.
struct Args {
    Dims d;
    int B, n, NI;           // n: rows per sequence in q, k, v, out; NI: intervals of n tokens
    uint64_t hash;          // configuration hash the state header must carry
    const int32_t* seqn;    // device [B]: tokens of each sequence (<= n), or null: n for all
    unsigned char* state;
    unsigned char* ws;
    const void* q;
    const void* k;
    const void* v;
    void* out;
    StateLayout sl;
    WsLayout wl;
};

// The state header was written by lola_init_state for this configuration and
// batch, and no earlier call marked the state faulted.  Kernels that advance or
// read a state test this first and, if it fails, return without writing anything,
// so a state meant for another configuration is never read or written with this
// one's layout.  (The fields are read with uniform addresses, so every wave of a
// workgroup takes the same branch as long as no other workgroup of the same launch
// writes the header; only the split scan does, and it broadcasts its test.)
__device__ __forceinline__ bool state_ok(const Args& a, bool allow_faulted = false)
{
    // the 32 header bytes in one load, and no early exit between the tests: the
    // fields are requested together instead of one round trip after another
    const StateHeader h = *(const StateHeader*)a.state;
    return (h.magic == kMagic) & (h.version == kVersion) & (h.cfg_hash == a.hash) & (h.batch == a.B) &
           (allow_faulted | (h.fault == 0));
}

// Tokens sequence b consumes in this call: its entry of the per-sequence counts
// clamped to [0, n], or n when the call has none.
__device__ __forceinline__ int seq_tokens(const Args& a, int b)
{
    if (!a.seqn) return a.n;
    const int v = a.seqn[b];
    return v < 0 ? 0 : (v > a.n ? a.n : v);
}

}  // namespace lola
