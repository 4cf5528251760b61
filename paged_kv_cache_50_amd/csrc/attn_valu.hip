// General paged attention kernel on the vector ALUs (gfx950).
//
// Computes, for one query row, the query heads of one kv-head chunk and one
// key partition, the online-softmax attention over the row's cached tokens
// reached through its block-table row (vLLM book, ch. 6 "Flux des paramètres
// du chemin non-cascadé": cu_seqlens_q, seqused_k, block_table).  Takes
// float32, bfloat16 and binary16 caches.  Used for float32 caches, for MHA
// decode (one query head per kv head, where the work is a matrix-vector
// product and matrix cores would idle) and as the generic varlen path.
//
// Work decomposition
//   grid.x = kv head * head chunks, grid.y = sequence (or query row in
//   kModeVarlenRows; plus z_base for launches split along this axis),
//   grid.z = key partition (slowest, so that the empty partitions of short
//   sequences dispatch last).  A workgroup is 4 waves of 64 lanes.
//   One token row of one kv head (head_size elements) is read by LPR lanes
//   with one 16-byte load each: 16 lanes for bf16 x 128, so a wave load
//   covers RPW = 64 / LPR consecutive tokens of one block, fully coalesced.
//   A wave step is NLS such loads; waves take steps round-robin.
//   Each row of LPR lanes keeps its own online-softmax state (running max m,
//   running sum l, fp32 accumulator) over the tokens it sees, so the hot loop
//   needs only the in-row dot-product reduction (DPP); the 4*RPW states are
//   merged once at the end (shuffles inside a wave, LDS across waves).
//   Block ids are read with wave-uniform (scalar) loads one step ahead; the
//   next step's K/V loads are issued before the current step is computed.
//   Tokens past the partition end are loaded from a clamped, in-bounds slot
//   and removed by select (never by multiply), so stale NaNs in unused slots
//   cannot leak into the result.
#include "device_common.h"
#include "pkv_internal.h"
#include "attn_common.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kNls = 4;  // 16-byte loads per lane per wave step (K and V each)

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
};
template <>
struct Elem<uint16_t> {
  static constexpr int kBytes = 2;
};
template <>
struct Elem<_Float16> {
  static constexpr int kBytes = 2;
};

// Dot product of a 16-byte K fragment with the query fragment of one head.
template <typename T>
__device__ __forceinline__ float frag_dot(const u32x4& k, const u32x4& q);

template <>
__device__ __forceinline__ float frag_dot<float>(const u32x4& k, const u32x4& q) {
  float s = __uint_as_float(k[0]) * __uint_as_float(q[0]);
  s = fmaf(__uint_as_float(k[1]), __uint_as_float(q[1]), s);
  s = fmaf(__uint_as_float(k[2]), __uint_as_float(q[2]), s);
  s = fmaf(__uint_as_float(k[3]), __uint_as_float(q[3]), s);
  return s;
}

template <>
__device__ __forceinline__ float frag_dot<uint16_t>(const u32x4& k, const u32x4& q) {
  // bf16 pairs, products exact, fp32 accumulation.
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k[w]), as_bf16x2(q[w]), s, false);
  return s;
}

template <>
__device__ __forceinline__ float frag_dot<_Float16>(const u32x4& k, const u32x4& q) {
  // binary16 pairs, products exact, fp32 accumulation.
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) s = __builtin_amdgcn_fdot2(as_f16x2(k[w]), as_f16x2(q[w]), s, false);
  return s;
}

// Widen a 16-byte V fragment to fp32 (4 or 8 values).
template <typename T>
__device__ __forceinline__ void frag_widen(const u32x4& v, float* out);

template <>
__device__ __forceinline__ void frag_widen<float>(const u32x4& v, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
}

template <>
__device__ __forceinline__ void frag_widen<uint16_t>(const u32x4& v, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = bf16_lo(v[i]);
    out[2 * i + 1] = bf16_hi(v[i]);
  }
}

template <>
__device__ __forceinline__ void frag_widen<_Float16>(const u32x4& v, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = f16_lo(v[i]);
    out[2 * i + 1] = f16_hi(v[i]);
  }
}

template <typename T>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v);
template <>
__device__ __forceinline__ void store_out<float>(void* out, int64_t idx, float v) {
  static_cast<float*>(out)[idx] = v;
}
template <>
__device__ __forceinline__ void store_out<uint16_t>(void* out, int64_t idx, float v) {
  static_cast<uint16_t*>(out)[idx] = static_cast<uint16_t>(f32_to_bf16_rne(v));
}
template <>
__device__ __forceinline__ void store_out<_Float16>(void* out, int64_t idx, float v) {
  static_cast<uint16_t*>(out)[idx] = static_cast<uint16_t>(f32_to_f16_rne(v));
}

template <typename T, int D, int BS, int GT>
__global__ void __launch_bounds__(kThreads) attn_valu_kernel(const AttnArgs a) {
  constexpr int E = Elem<T>::kBytes;
  constexpr int EPL = 16 / E;       // elements per lane per load
  constexpr int LPR = D / EPL;      // lanes per token row
  constexpr int RPW = 64 / LPR;     // token rows per wave load
  constexpr int TPS = RPW * kNls;   // tokens per wave step
  static_assert(RPW <= BS && BS % RPW == 0, "a wave load must stay inside one block");
  static_assert(LPR >= 4 && LPR <= 64, "row width");

  __shared__ float s_acc[kWaves][GT][D];
  __shared__ float s_m[kWaves][GT];
  __shared__ float s_l[kWaves][GT];

  Item it;
  if (!resolve_item(a, blockIdx.y + a.z_base, it)) return;
  const int part = blockIdx.z;  // partitions on the slowest axis: empty ones dispatch last
  if (part >= it.nparts) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPR;
  const int c = lane % LPR;
  const int group = a.num_heads / a.num_kv_heads;
  // one column per kv head: adjacent heads swap columns (column_head)
  const int kvh = a.head_chunks == 1 ? column_head(blockIdx.x, a.num_kv_heads, D * E)
                                     : blockIdx.x / a.head_chunks;
  const int h0 = kvh * group + (blockIdx.x % a.head_chunks) * GT;

  const int pstart = it.base + part * it.P;
  const int pend = min(pstart + it.P, it.L_end);
  const int pbegin = it.L_begin;                 // first visible key (sliding window)

  // query fragments of the chunk's heads
  u32x4 qf[GT];
  const T* qrow = static_cast<const T*>(a.q) + ((int64_t)it.row * a.num_heads + h0) * D + c * EPL;
#pragma unroll
  for (int h = 0; h < GT; ++h) qf[h] = *reinterpret_cast<const u32x4*>(qrow + (int64_t)h * D);

  float m[GT], l[GT], acc[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  // the cascade prefix pass reads every row's keys through block-table row 0
  const int bt_row = a.mode == kModePrefix ? 0 : it.seq;
  const int32_t* __restrict__ bt = a.block_tables + (int64_t)bt_row * a.max_blocks_per_seq;
  const T* __restrict__ kc = static_cast<const T*>(a.k_cache);
  const T* __restrict__ vc = static_cast<const T*>(a.v_cache);
  const int64_t tok_stride = (int64_t)a.num_kv_heads * D;            // elements between tokens
  const int64_t lane_off = (int64_t)kvh * D + c * EPL + r * tok_stride;
  const int64_t max_blk = a.num_blocks - 1;
  const int nsteps = (pend > pstart) ? (pend - pstart + TPS - 1) / TPS : 0;

  u32x4 kA[kNls], vA[kNls], kB[kNls], vB[kNls];   // ping-pong step buffers

  // Block ids of one wave step (wave uniform, scalar loads), fetched one
  // step early so that issuing a step's loads never waits on them.  A step
  // spans NBS blocks; a load covers RPW consecutive tokens inside one block.
  constexpr int NBS = TPS > BS ? TPS / BS : 1;
  const int last_bi = (pend - 1) / BS;
  auto fetch_ids = [&](int step, int64_t* ids) {
    const int t0 = pstart + step * TPS;
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
      const int bi = __builtin_amdgcn_readfirstlane(min(t0 / BS + b, last_bi));
      ids[b] = min((int64_t)max(load_uniform_i32(bt, bi), 0), max_blk) * a.block_stride;
    }
  };
  // Tokens past the partition end read a slot of a valid block (in bounds).
  auto issue = [&](int step, const int64_t* ids, u32x4* kr, u32x4* vr) {
#pragma unroll
    for (int i = 0; i < kNls; ++i) {
      const int t0 = pstart + step * TPS + i * RPW;                  // wave uniform
      const int64_t off = ids[(i * RPW) / BS] + (int64_t)(t0 % BS) * tok_stride + lane_off;
      kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kc + off));
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vc + off));
    }
  };

  auto compute = [&](int step, const u32x4* K, const u32x4* V) {
    const int tbase = pstart + step * TPS + r;
    float s[kNls][GT];
#pragma unroll
    for (int i = 0; i < kNls; ++i) {
      const bool valid = tbase + i * RPW < pend && tbase + i * RPW >= pbegin;
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float d = group_sum<LPR>(frag_dot<T>(K[i], qf[h]));
        s[i][h] = valid ? d * a.scale_log2 : -INFINITY;
      }
    }
    float vf[kNls][EPL];
#pragma unroll
    for (int i = 0; i < kNls; ++i) {
      const bool valid = tbase + i * RPW < pend && tbase + i * RPW >= pbegin;
      frag_widen<T>(V[i], vf[i]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) vf[i][e] = valid ? vf[i][e] : 0.f;
    }
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int i = 1; i < kNls; ++i) mx = fmaxf(mx, s[i][h]);
      const float mn = fmaxf(m[h], mx);
      const float mref = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = fast_exp2(m[h] - mref);
      float p[kNls];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < kNls; ++i) {
        p[i] = fast_exp2(s[i][h] - mref);
        psum += p[i];
      }
      l[h] = l[h] * alpha + psum;
      m[h] = mn;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float o = acc[h][e] * alpha;
#pragma unroll
        for (int i = 0; i < kNls; ++i) o = fmaf(p[i], vf[i][e], o);
        acc[h][e] = o;
      }
    }
  };

  // Two steps in flight per wave; buffers alternate instead of being copied.
  int64_t ids[NBS];
  int step = wave;
  if (step < nsteps) {
    fetch_ids(step, ids);
    issue(step, ids, kA, vA);
    if (step + kWaves < nsteps) fetch_ids(step + kWaves, ids);
  }
  while (step < nsteps) {
    if (step + kWaves < nsteps) {
      issue(step + kWaves, ids, kB, vB);
      if (step + 2 * kWaves < nsteps) fetch_ids(step + 2 * kWaves, ids);
    }
    compute(step, kA, vA);
    step += kWaves;
    if (step >= nsteps) break;
    if (step + kWaves < nsteps) {
      issue(step + kWaves, ids, kA, vA);
      if (step + 2 * kWaves < nsteps) fetch_ids(step + 2 * kWaves, ids);
    }
    compute(step, kB, vB);
    step += kWaves;
  }

  // Merge the RPW row states of this wave (rows are LPR lanes apart).
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    float M = m[h];
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float Mref = (M == -INFINITY) ? 0.f : M;
    const float f = fast_exp2(m[h] - Mref);
    float lh = l[h] * f;
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) lh += __shfl_xor(lh, o);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = acc[h][e] * f;
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) v += __shfl_xor(v, o);
      acc[h][e] = v;
    }
    m[h] = M;
    l[h] = lh;
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][h][c * EPL + e] = acc[h][e];
      if (c == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // Merge the waves and write the row (or this partition's partial result).
  for (int idx = threadIdx.x; idx < GT * D; idx += kThreads) {
    const int h = idx / D;
    const int d = idx % D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    const float Mref = (M == -INFINITY) ? 0.f : M;
    float O = 0.f, Ls = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(s_m[w][h] - Mref);
      O = fmaf(s_acc[w][h][d], f, O);
      Ls = fmaf(s_l[w][h], f, Ls);
    }
    const int head = h0 + h;
    if (it.nranges == 1 && a.mode != kModePrefix) {
      const float v = Ls > 0.f ? O / Ls : 0.f;
      store_out<T>(a.out, ((int64_t)it.row * a.num_heads + head) * D + d, v);
      if (d == 0 && a.lse_out)
        a.lse_out[(int64_t)it.row * a.num_heads + head] =
            Ls > 0.f ? (M + acc_log2(Ls)) * kLn2 : -INFINITY;
    } else {
      const int64_t widx = ((int64_t)part * a.num_heads + head) * a.num_seqs + it.seq;
      a.ws_o[widx * D + d] = Ls > 0.f ? O / Ls : 0.f;
      if (d == 0) a.ws_lse[widx] = Ls > 0.f ? M + acc_log2(Ls) : -INFINITY;
    }
  }
}

}  // namespace

template <typename T, int D, int BS>
static hipError_t launch_gt(const AttnArgs& a, int gt, dim3 grid, hipStream_t st) {
  switch (gt) {
    case 1: hipLaunchKernelGGL((attn_valu_kernel<T, D, BS, 1>), grid, dim3(kThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((attn_valu_kernel<T, D, BS, 2>), grid, dim3(kThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL((attn_valu_kernel<T, D, BS, 4>), grid, dim3(kThreads), 0, st, a); break;
    case 8: hipLaunchKernelGGL((attn_valu_kernel<T, D, BS, 8>), grid, dim3(kThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_bs(const AttnArgs& a, int bs, int gt, dim3 grid, hipStream_t st) {
  switch (bs) {
    case 8: return launch_gt<T, D, 8>(a, gt, grid, st);
    case 16: return launch_gt<T, D, 16>(a, gt, grid, st);
    case 32: return launch_gt<T, D, 32>(a, gt, grid, st);
    case 64: return launch_gt<T, D, 64>(a, gt, grid, st);
    case 128: return launch_gt<T, D, 128>(a, gt, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_valu(const AttnArgs& a, int dtype, int head_size, int block_size,
                            int heads_per_chunk, dim3 grid, hipStream_t stream) {
  auto by_head = [&](auto elem) -> hipError_t {
    using T = decltype(elem);
    switch (head_size) {
      case 64: return launch_bs<T, 64>(a, block_size, heads_per_chunk, grid, stream);
      case 128: return launch_bs<T, 128>(a, block_size, heads_per_chunk, grid, stream);
      case 256: return launch_bs<T, 256>(a, block_size, heads_per_chunk, grid, stream);
      default: return hipErrorInvalidValue;
    }
  };
  if (dtype == PKV_F32) return by_head(float{});
  if (dtype == PKV_BF16) return by_head(uint16_t{});
  if (dtype == PKV_F16) return by_head(_Float16{});
  return hipErrorInvalidValue;
}

}  // namespace pkv
