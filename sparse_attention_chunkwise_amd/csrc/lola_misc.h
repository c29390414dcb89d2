// State initialisation and read-out kernels.
#pragma once

#include "lola_prefill.h"

namespace lola {

// Zero every chain block, write the header and copy W.  grid (B*Hkv + 1).
__global__ __launch_bounds__(256) void init_kernel(Args a, const float* W, uint64_t cfg_hash)
{
    const int blk = blockIdx.x;
    if (blk == (int)gridDim.x - 1) {
        // the whole 256-byte header block, padding included, so that two states that
        // saw the same calls are equal byte for byte
        if (threadIdx.x < 64) ((uint32_t*)a.state)[threadIdx.x] = 0u;
        __syncthreads();
        if (threadIdx.x == 0) {
            StateHeader* h = (StateHeader*)a.state;
            h->magic = kMagic;
            h->version = kVersion;
            h->cfg_hash = cfg_hash;
            h->batch = a.B;
            h->fault = 0;
        }
        float* Wd = (float*)(a.state + a.sl.W);
        const size_t nw = (size_t)a.d.Hkv * a.d.Fh * a.d.D;
        uint16_t* Wb = (uint16_t*)(a.state + a.sl.Wb);
        const size_t per = (size_t)a.d.Fh * a.d.D;
        for (size_t i = threadIdx.x; i < nw; i += 256) {
            const float x = W[i];
            Wd[i] = x;
            const uint16_t h = __builtin_bit_cast(uint16_t, (__bf16)x);
            const float r1 = x - __uint_as_float((uint32_t)h << 16);
            const uint16_t m = __builtin_bit_cast(uint16_t, (__bf16)r1);
            const size_t gi = i / per, r = i % per;
            Wb[(3 * gi) * per + r] = h;
            Wb[(3 * gi + 1) * per + r] = m;
            Wb[(3 * gi + 2) * per + r] = __builtin_bit_cast(uint16_t, (__bf16)(r1 - __uint_as_float((uint32_t)m << 16)));
        }
        return;
    }
    uint32_t* p = (uint32_t*)(a.state + a.sl.chains + (size_t)blk * a.sl.chain_bytes);
    const size_t nwords = a.sl.chain_bytes / 4;
    for (size_t i = threadIdx.x; i < nwords; i += 256) p[i] = 0u;
}

// Copy one chain's memories out, cache in ascending position order.
// grid (B*Hkv), block 256.
template <typename T>
__global__ __launch_bounds__(256) void read_cache_kernel(Args a, int32_t* count, int64_t* pos, T* k_out, T* v_out,
                                                         float* H_out, float* s_out, int64_t* tokens_seen)
{
    if (!state_ok(a, true)) return;  // header mismatch: the outputs are not written (a faulted state is read)
    const int chain = blockIdx.x, b = chain / a.d.Hkv, g = chain % a.d.Hkv;
    const int D = a.d.D, F = a.d.F, C = a.d.C;
    Chain ch = chain_of(a, chain);
    const int cnt = min(max(ch.cnt(), 0), C);
    const int32_t* cp = ch.cpos();
    if (threadIdx.x == 0) {
        if (count) count[chain] = cnt;
        if (tokens_seen && g == 0) tokens_seen[b] = ch.tok();
    }
    for (int i = threadIdx.x; i < C; i += 256) {
        int dst = i;
        if (i < cnt) {
            int rank = 0;
            for (int j = 0; j < cnt; ++j) rank += cp[j] < cp[i];
            dst = rank;
            if (pos) pos[(size_t)chain * C + dst] = cp[i];
        } else if (pos) {
            pos[(size_t)chain * C + i] = -1;
        }
        for (int j = 0; j < D; ++j) {
            if (k_out) k_out[((size_t)chain * C + dst) * D + j] = i < cnt ? ch.cache_k<T>()[(size_t)i * D + j] : from_f32<T>(0.f);
            if (v_out) v_out[((size_t)chain * C + dst) * D + j] = i < cnt ? ch.cache_v<T>()[(size_t)i * D + j] : from_f32<T>(0.f);
        }
    }
    if (H_out)
        for (int i = threadIdx.x; i < F * D; i += 256) H_out[(size_t)chain * F * D + i] = ch.H()[(i % D) * F + i / D];
    if (s_out)
        for (int i = threadIdx.x; i < F; i += 256) s_out[(size_t)chain * F + i] = ch.s()[i];
}

}  // namespace lola
