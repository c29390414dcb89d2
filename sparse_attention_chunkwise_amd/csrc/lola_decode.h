// Decode step of the LoLA layer (gfx950): one one-token update interval for
// every (sequence, KV head) chain in a single fused launch, read and write of
// the state in place.  grid (B*Hkv), block 256.
//
// Per chain, with t = tokens seen:
//   read    -- the G query heads of the chain attend with exact softmax to the
//              window [t-w+1, t] (ring + the new token) and to the cache, and
//              linearly to the state (H, s) and to the key at t-w that leaves
//              the window at this step (the new token itself when w = 0);
//              one shared denominator (LoLA summary, "Inferentiestrategie",
//              step 4);
//   manage  -- that leaving key and the cached keys are scored with the SRE
//              equation ("Het Self-Recall Error (SRE) Mechanisme") against the
//              step-start state; if they exceed the capacity the lowest
//              (SRE ascending, newest first) is folded into H, s by an outer
//              product and the leaving key takes its cache slot (steps 1-3).
#pragma once

#include "lola_prefill.h"

namespace lola {

struct DecodeSmem {
    size_t H, s, W, q, phq, lg, acc, misc, phf, kv, total;
};

__host__ __device__ inline DecodeSmem decode_smem(int D, int F, int G, int C)
{
    DecodeSmem m;
    int Fh = F / 2;
    size_t off = 0;
    m.H = off;    off += sizeof(float) * (size_t)F * (D + 4);
    m.s = off;    off += sizeof(float) * F;
    m.W = off;    off += sizeof(float) * (size_t)Fh * (D + 1);
    m.q = off;    off += sizeof(float) * (size_t)G * D;
    m.phq = off;  off += sizeof(float) * (size_t)G * F;
    m.lg = off;   off += sizeof(float) * (size_t)G * 256;
    m.acc = off;  off += sizeof(float) * (size_t)G * D;
    m.misc = off; off += sizeof(float) * (size_t)(4 * G + C + 64);
    m.phf = off;  off += sizeof(float) * F;
    m.kv = off;   off += sizeof(float) * 2 * D;
    m.total = align_up(off, 16);
    return m;
}

template <int D, int F, typename T>
__global__ __launch_bounds__(256) void decode_kernel(Args a)
{
    constexpr int NW = 4, HP = D + 4, Fh = F / 2, NH = F / 4;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    if (!state_ok(a)) return;  // header mismatch or faulted state: nothing is read or written
    const Dims& d = a.d;
    const int G = d.G, w = d.w, C = d.C;
    const DecodeSmem sm = decode_smem(D, F, G, C);
    float* Hs = (float*)(smem + sm.H);
    float* ss = (float*)(smem + sm.s);
    float* Ws = (float*)(smem + sm.W);      // [Fh][D+1]
    float* qs = (float*)(smem + sm.q);      // [G][D]
    float* phq = (float*)(smem + sm.phq);   // [G][F]
    float* lgs = (float*)(smem + sm.lg);    // [G][256]
    float* acc = (float*)(smem + sm.acc);   // [G][D]
    float* misc = (float*)(smem + sm.misc); // mrun[G], Z[G], zlin[G], kap[G], esc[C+1], ...
    float* phf = (float*)(smem + sm.phf);   // phi of the folded / pending key
    float* kvs = (float*)(smem + sm.kv);    // pending key [D], value [D]
    float* mrun = misc;
    float* Zs = misc + G;
    float* zlin = misc + 2 * G;
    float* kap = misc + 3 * G;
    float* esc = misc + 4 * G;              // [C+1]
    __shared__ unsigned long long red[NW];
    __shared__ int sel[2];

    const int chain = blockIdx.x, b = chain / d.Hkv, g = chain % d.Hkv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, qg = lane >> 4;
    Chain ch = chain_of(a, chain);
    const int64_t t = ch.tok();
    const int cnt = min(max(ch.cnt(), 0), C);
    const T* knew = (const T*)a.k + ((size_t)b * d.Hkv + g) * D;
    const T* vnew = (const T*)a.v + ((size_t)b * d.Hkv + g) * D;
    // the key leaving the window at this step: position t - w (ring slot t % w),
    // or the new token itself when there is no window
    const bool hasE = (w == 0) || (t - w >= 0);
    const int64_t pE = t - w;
    const T* kE = w == 0 ? knew : ch.ring_k<T>() + (size_t)(t % (w > 0 ? w : 1)) * D;
    const T* vE = w == 0 ? vnew : ch.ring_v<T>() + (size_t)(t % (w > 0 ? w : 1)) * D;

    // ---- load state, W, queries, the leaving pair ----
    for (int i = tid; i < F * D; i += 256) Hs[(i % F) * HP + (i / F)] = ch.H()[i];  // state H is [D][F]
    for (int i = tid; i < F; i += 256) ss[i] = ch.s()[i];
    const float* W = (const float*)(a.state + a.sl.W) + (size_t)g * Fh * D;
    for (int i = tid; i < Fh * D; i += 256) Ws[(i / D) * (D + 1) + (i % D)] = W[i];
    for (int i = tid; i < G * D; i += 256) {
        const int hh = i / D, j = i % D;
        qs[i] = to_f32(((const T*)a.q)[((size_t)b * d.Hq + g * G + hh) * D + j]);
        acc[i] = 0.f;
    }
    for (int j = tid; j < D; j += 256) {
        kvs[j] = hasE ? to_f32(kE[j]) : 0.f;
        kvs[D + j] = hasE ? to_f32(vE[j]) : 0.f;
    }
    if (tid < G) { mrun[tid] = 0.f; Zs[tid] = 0.f; }
    __syncthreads();

    // ---- phi of the G queries (rows 0..G-1) and of the leaving key (row G) ----
    for (int row = wave; row <= G; row += NW) {
        const float* x = row < G ? qs + row * D : kvs;
        float z = 0.f;
        if (lane < Fh)
            for (int j = 0; j < D; ++j) z += Ws[lane * (D + 1) + j] * x[j];
        float zmax = wave_max(lane < Fh ? z : -INFINITY);
        float zmin = -wave_max(lane < Fh ? -z : -INFINITY);
        float ep = lane < Fh ? expf(z - zmax) : 0.f;
        float en = lane < Fh ? expf(zmin - z) : 0.f;
        float sp = wave_sum(ep), sn = wave_sum(en);
        float* o = row < G ? phq + row * F : phf;
        if (lane < Fh) { o[lane] = ep / sp; o[Fh + lane] = en / sn; }
    }
    __syncthreads();

    // ---- linear read: H^T phi(q), s . phi(q), plus the leaving key (kappa) ----
    if (tid < G) {
        float z = 0.f, kp = 0.f;
        for (int f = 0; f < F; ++f) { z += phq[tid * F + f] * ss[f]; kp += phq[tid * F + f] * phf[f]; }
        kap[tid] = hasE ? kp : 0.f;
        zlin[tid] = z + kap[tid];
    }
    __syncthreads();

    // ---- softmax keys: window [max(0,t-w+1), t] then cache slots; chunks of 256 ----
    const int64_t ws0 = t - w + 1 > 0 ? t - w + 1 : 0;
    const int nWin = w > 0 ? (int)(t - ws0 + 1) : 0;
    const int nKey = nWin + cnt;
    auto keyk = [&](int j) -> const T* {
        if (j < nWin) {
            const int64_t p = ws0 + j;
            return p == t ? knew : ch.ring_k<T>() + (size_t)(p % w) * D;
        }
        return ch.cache_k<T>() + (size_t)(j - nWin) * D;
    };
    auto keyv = [&](int j) -> const T* {
        if (j < nWin) {
            const int64_t p = ws0 + j;
            return p == t ? vnew : ch.ring_v<T>() + (size_t)(p % w) * D;
        }
        return ch.cache_v<T>() + (size_t)(j - nWin) * D;
    };
    for (int kb = 0; kb < nKey; kb += 256) {
        const int nk = nKey - kb < 256 ? nKey - kb : 256;
        if (tid < nk) {
            const T* kr = keyk(kb + tid);
            float kreg[D];
#pragma unroll
            for (int j = 0; j < D; ++j) kreg[j] = to_f32(kr[j]);
            for (int hh = 0; hh < G; ++hh) {
                float dot = 0.f;
#pragma unroll
                for (int j = 0; j < D; ++j) dot += qs[hh * D + j] * kreg[j];
                lgs[hh * 256 + tid] = d.tau * dot;
            }
        }
        __syncthreads();
        if (tid < G) {
            float mx = mrun[tid];
            for (int j = 0; j < nk; ++j) mx = fmaxf(mx, lgs[tid * 256 + j]);
            const float resc = expf(mrun[tid] - mx);
            float z = Zs[tid] * resc;
            for (int j = 0; j < nk; ++j) {
                const float p = expf(lgs[tid * 256 + j] - mx);
                lgs[tid * 256 + j] = p;
                z += p;
            }
            kap[tid] = resc;  // reuse as the rescale factor of this chunk
            Zs[tid] = z;
            mrun[tid] = mx;
        }
        __syncthreads();
        for (int i = tid; i < G * D; i += 256) {
            const int hh = i / D, j = i % D;
            float o = acc[i] * kap[hh];
            for (int k2 = 0; k2 < nk; ++k2) o += lgs[hh * 256 + k2] * to_f32(keyv(kb + k2)[j]);
            acc[i] = o;
        }
        __syncthreads();
    }
    // ---- combine and store ----
    for (int i = tid; i < G * D; i += 256) {
        const int hh = i / D, j = i % D;
        float lin = 0.f;
        for (int f = 0; f < F; ++f) lin += phq[hh * F + f] * Hs[f * HP + j];
        if (hasE) {
            float kp = 0.f;
            for (int f = 0; f < F; ++f) kp += phq[hh * F + f] * phf[f];
            lin += kp * kvs[D + j];
        }
        const float el = expf(-mrun[hh]);
        const float o = (acc[i] + el * lin) / (Zs[hh] + el * zlin[hh]);
        ((T*)a.out)[((size_t)b * d.Hq + g * G + hh) * D + j] = from_f32<T>(o);
    }

    // ---- SRE of cache slots [0, cnt) and the leaving key (index cnt) ----
    const int nU = cnt + (hasE ? 1 : 0);
    auto candk = [&](int u) -> const T* { return u < cnt ? ch.cache_k<T>() + (size_t)u * D : kE; };
    auto candv = [&](int u) -> const T* { return u < cnt ? ch.cache_v<T>() + (size_t)u * D : vE; };
    for (int tile = wave; tile * 16 < nU; tile += NW) {
        const int u = tile * 16 + r16;
        const bool uv = u < nU;
        // z^T = W . K^T over 16 candidates (f32 MFMA)
        float kreg[D / 4];
        {
            const T* kr = candk(uv ? u : 0) + qg * (D / 4);
#pragma unroll
            for (int m = 0; m < D / 4; ++m) kreg[m] = uv ? to_f32(kr[m]) : 0.f;
        }
        floatx4 zt[Fh / 16];
#pragma unroll
        for (int ft = 0; ft < Fh / 16; ++ft) {
            zt[ft] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < D / 4; ++m)
                zt[ft] = __builtin_amdgcn_mfma_f32_16x16x4f32(Ws[(ft * 16 + r16) * (D + 1) + qg * (D / 4) + m], kreg[m],
                                                               zt[ft], 0, 0, 0);
        }
        float zmax = -INFINITY, zmin = INFINITY;
#pragma unroll
        for (int ft = 0; ft < Fh / 16; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) { zmax = fmaxf(zmax, zt[ft][i]); zmin = fminf(zmin, zt[ft][i]); }
        zmax = quad_max(zmax);
        zmin = quad_min(zmin);
        float hk[NH];
        float sp = 0.f, sn = 0.f;
#pragma unroll
        for (int ft = 0; ft < Fh / 16; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e1 = expf(zt[ft][i] - zmax), e2 = expf(zmin - zt[ft][i]);
                hk[ft * 4 + i] = e1;
                hk[NH / 2 + ft * 4 + i] = e2;
                sp += e1;
                sn += e2;
            }
        sp = quad_sum(sp);
        sn = quad_sum(sn);
#pragma unroll
        for (int j = 0; j < NH / 2; ++j) { hk[j] /= sp; hk[NH / 2 + j] /= sn; }
        float dd = 0.f;
#pragma unroll
        for (int j = 0; j < NH; ++j) dd += hk[j] * ss[held_feature<Fh>(qg, j)];
        dd = quad_sum(dd);
        // n^T = H^T phi^T ; error over the lane's d rows
        const T* vr = candv(uv ? u : 0);
        float e = 0.f;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            floatx4 nt = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mf = 0; mf < NH; ++mf)
                nt = __builtin_amdgcn_mfma_f32_16x16x4f32(Hs[held_feature<Fh>(qg, mf) * HP + dt * 16 + r16], hk[mf], nt,
                                                          0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float rr = dd > 0.f ? nt[i] / dd : 0.f;
                const float df = rr - (uv ? to_f32(vr[dt * 16 + qg * 4 + i]) : 0.f);
                e += df * df;
            }
        }
        e = quad_sum(e);
        if (qg == 0 && uv) esc[u] = e;
    }
    __syncthreads();

    // ---- pick the pair to fold: lowest SRE, newest position on a tie ----
    int victim = -1;
    if (hasE && nU > C) {
        unsigned long long best = ~0ull;
        for (int u = tid; u < nU; u += 256) {
            const uint32_t pos = u < cnt ? (uint32_t)ch.cpos()[u] : (uint32_t)pE;
            const unsigned long long key = ((unsigned long long)__float_as_uint(esc[u]) << 32) | (0xffffffffu - pos);
            best = key < best ? key : best;
        }
        for (int o = 32; o > 0; o >>= 1) {
            unsigned long long other = __shfl_xor(best, o, 64);
            best = other < best ? other : best;
        }
        if (lane == 0) red[wave] = best;
        __syncthreads();
        if (tid == 0) {
            unsigned long long bb = red[0];
            for (int i = 1; i < NW; ++i) bb = red[i] < bb ? red[i] : bb;
            const uint32_t pos = 0xffffffffu - (uint32_t)(bb & 0xffffffffu);
            int vi = cnt;  // the leaving key unless a cache slot holds that position
            for (int u = 0; u < cnt; ++u)
                if ((uint32_t)ch.cpos()[u] == pos) vi = u;
            sel[0] = vi;
        }
        __syncthreads();
        victim = sel[0];
    }

    // ---- fold the victim: H += phi(k) v^T, s += phi(k) ----
    if (victim >= 0) {
        if (victim < cnt) {
            // phi of the evicted cache key (the leaving key's phi is already in phf)
            const T* kr = candk(victim);
            for (int j = tid; j < D; j += 256) kvs[j] = to_f32(kr[j]);
            __syncthreads();
            if (wave == 0) {
                float z = 0.f;
                if (lane < Fh)
                    for (int j = 0; j < D; ++j) z += Ws[lane * (D + 1) + j] * kvs[j];
                float zmax = wave_max(lane < Fh ? z : -INFINITY);
                float zmin = -wave_max(lane < Fh ? -z : -INFINITY);
                float ep = lane < Fh ? expf(z - zmax) : 0.f;
                float en = lane < Fh ? expf(zmin - z) : 0.f;
                float sp = wave_sum(ep), sn = wave_sum(en);
                if (lane < Fh) { phf[lane] = ep / sp; phf[Fh + lane] = en / sn; }
            }
            __syncthreads();
        }
        const T* vr = candv(victim);
        for (int i = tid; i < F * D; i += 256) {
            const int f = i % F, j = i / F;
            ch.H()[i] = Hs[f * HP + j] + phf[f] * to_f32(vr[j]);
        }
        for (int f = tid; f < F; f += 256) ch.s()[f] = ss[f] + phf[f];
    }
    __syncthreads();

    // ---- cache slot update, then the ring (the leaving pair lives in slot t % w) ----
    int slot = -1;
    if (hasE) {
        if (nU <= C) slot = cnt;
        else if (victim < cnt) slot = victim;
    }
    if (slot >= 0) {
        for (int j = tid; j < D; j += 256) {
            ch.cache_k<T>()[(size_t)slot * D + j] = kE[j];
            ch.cache_v<T>()[(size_t)slot * D + j] = vE[j];
        }
    }
    __syncthreads();
    if (w > 0) {
        const int rs = (int)(t % w);
        for (int j = tid; j < D; j += 256) {
            ch.ring_k<T>()[(size_t)rs * D + j] = knew[j];
            ch.ring_v<T>()[(size_t)rs * D + j] = vnew[j];
        }
    }
    if (tid == 0) {
        if (slot >= 0) ch.cpos()[slot] = (int32_t)pE;
        if (hasE && nU <= C) ch.cnt() = cnt + 1;
        ch.tok() = t + 1;
    }
}

}  // namespace lola
