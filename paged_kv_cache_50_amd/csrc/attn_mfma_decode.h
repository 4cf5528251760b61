// Grouped-query paged decode attention on the matrix cores (gfx950 MFMA).
//
// With GQA the query heads of one kv-head group read the same K/V rows, so
// for each tile of cached tokens the work is a small dense contraction: the
// logits of g query heads against 32 keys, then the g probability rows
// against the 32 value rows (vLLM book, ch. 6 "Flux des paramètres du chemin
// non-cascadé": one kernel gathering K/V through the block table).  Each kv
// head's K/V tile is loaded once and shared by the group's query heads.
//
// Layout (v_mfma_f32_16x16x32_bf16, or _f16 over binary16 caches; N = 16
// query-head columns, g <= 16 used):
//   S^T[32 tok x 16 heads] = K[32 x 128] . Q^T[128 x 16]: the K tile is read
//     from HBM as whole 256-byte token rows (16 lanes x 16 bytes per row, the
//     most efficient gather pattern), staged in LDS with an XOR swizzle of the
//     16-byte slots and read back as A operands (lane = token row, 8 dims),
//     conflict-free on both sides; Q^T is a B operand held in registers.
//   The S^T accumulator gives each lane 8 logits of ONE head column, so the
//   online-softmax max/sum need only two cross-lane steps (permlane swaps
//   across the 4 token groups), and the probabilities are already laid out as
//   the B operand P^T of the second product.
//   O^T[128 x 16] += V^T[128 x 32] . P^T[32 x 16]: the V tile is written to LDS
//   in its natural token-major layout and read back transposed with
//   ds_read_b64_tr_b16, two reads per 16-dim tile.
//   O^T's accumulator column is again the lane's head, so the rescale by
//   exp(m_old - m_new) is a plain per-lane multiply.
// A workgroup (4 waves) owns one (sequence, kv-head chunk, range of
// consecutive key partitions); the grid puts ranges on its slowest axis so
// that the workgroups of ranges a short sequence does not have are dispatched
// last.  Either wave w owns partition w of a full 4-partition range, or the
// waves take the range's 32-token tiles round-robin.  A wave copies its
// tile's K rows from registers into its LDS area, issues the next tile's K
// loads into the same registers, computes the logits; then does the same
// with the V rows (in the same LDS area) and the PV product, so the next
// tile's loads are in flight while it computes and the LDS of a workgroup
// stays at 35 KiB (block ids run one tile further ahead).
// Head size 256 (16-bit caches): tiles of 16 tokens, so that a tile is the
// same 8 KiB and eight loads per lane; the logits take 8 k-steps of one
// 16-token block, and the PV product is the 16 x 16 x 16 form, whose A
// operand is a single transposed read.  The merge stages [16][256] floats
// per wave, so the workgroup's LDS is 65 KiB (still two per CU).  The 4 waves merge
// their softmax states through LDS at the end and write the row, or the
// range's partial result.
// Tokens past the partition end are loaded from an in-bounds slot of the last
// valid block; their logits are replaced by -inf and their V rows by zeros
// (select, never multiply), so stale NaNs in unused cache slots cannot reach
// the result.
#pragma once

#include <type_traits>

#include "attn_common.h"
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace dec {


constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// Lazy exponent reference: probabilities are formed against the running
// reference, which is raised (with a rescale of the accumulators) only when
// a tile's max outgrows it by more than kRescaleSlack (log2 units), so a
// probability never exceeds 2^kRescaleSlack.  It starts at a finite stand-in
// for -inf, far below any logit: the first visible key raises it, and a
// column that sees no key keeps it with sum 0.
constexpr float kRescaleSlack = 8.f;
constexpr float kSlackSum = 256.f;              // 2^kRescaleSlack
constexpr float kMinRef = -3.0e38f;

// Per-wave geometry for head size D (128 or 256).  A tile is 32 tokens at
// D = 128 and 16 at D = 256, so that it is 8 KiB of K (and of V) either way,
// eight 16-byte loads per lane.  A wave stages a tile's K rows, computes the
// logits, then stages the V rows in the same area; at the end the area holds
// the wave's [16 heads][D] float32 output for the merge.
template <int D>
struct Geo {
  static_assert(D == 128 || D == 256, "head size");
  static constexpr int kTile = D == 256 ? 16 : 32;        // tokens per wave step
  static constexpr int kVPitch = D * 2 + 16;              // LDS bytes per V token row (padded)
  static constexpr int kKTileBytes = kTile * D * 2;
  static constexpr int kVTileBytes = kTile * kVPitch;
  static constexpr int kTileArea = kKTileBytes > kVTileBytes ? kKTileBytes : kVTileBytes;
  static constexpr int kMergeBytes = 16 * D * 4;
  // 8.5 KiB per wave (34 KiB per workgroup, 35 KiB with the merge arrays) at
  // D = 128; 16 KiB (64 KiB, 65 KiB) at D = 256
  static constexpr int kWaveLds = kTileArea > kMergeBytes ? kTileArea : kMergeBytes;
};
// LDS of a workgroup whose waves cover HP kv heads each
template <int HP, int D = 128>
constexpr int kLdsBytesHp = HP * kWaves * Geo<D>::kWaveLds;
constexpr int kLdsBytes = kLdsBytesHp<1>;

__device__ __forceinline__ float xmax16_32(float x) {
  // max over the 4 lanes {l, l^16, l^32, l^48}: the token groups of a column
  auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = fmaxf(__int_as_float(p16[0]), __int_as_float(p16[1]));
  auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(p32[0]), __int_as_float(p32[1]));
}

__device__ __forceinline__ float xsum16_32(float x) {
  auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(p16[0]) + __int_as_float(p16[1]);
  auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(p32[0]) + __int_as_float(p32[1]);
}

// LDS byte offset of 16-byte chunk c (0..15) of token row t in a K tile:
// slots are XOR-swizzled by the row so that 16 lanes reading the same chunk
// of 16 different rows hit 16 different bank groups.
template <int D>
__device__ __forceinline__ int ktile_off(int t, int c) { return t * (D * 2) + ((c ^ (t & 15)) << 4); }

// FP8: the caches hold e4m3 codes with per-kv-head scales; a token row is
// then 128 bytes, read by 8 lanes, and converted (exactly) to bfloat16 while
// it is staged in LDS, so the matrix-core part is the same.  The K scale is
// folded into the logit scale and the V scale into the output.  With HP = 2
// a wave serves two adjacent kv heads: one load covers 4 tokens' 256-byte
// rows of both heads (16 lanes a row, the gather pattern of bfloat16 rows),
// each lane converts into the K or V tile of its head, and the products and
// softmax states run per head.
// DT is the cache's pkv_dtype: PKV_BF16, PKV_F16 (the products then take
// binary16 operands and the output is binary16) or PKV_FP8_E4M3.
// One workgroup's work: kv-head chunk bx (kv-head pair with HP = 2), row
// item zi (before the dispatch order is applied), key range bz of nz.  The
// caller provides the LDS areas (kLdsBytesHp<HP>, 16-byte aligned, and the
// two [kWaves][32] merge arrays).
template <int BS, int DT, int HP, int D = 128>
__device__ __forceinline__ void decode_block(const AttnArgs& a, int bx, int zi, int bz, int nz,
                                             char* __restrict__ s_lds, float (*s_m)[32],
                                             float (*s_l)[32]) {
  static_assert(BS == 8 || BS == 16 || BS == 32 || BS == 64 || BS == 128, "block size");
  static_assert(DT == PKV_BF16 || DT == PKV_F16 || DT == PKV_FP8_E4M3, "cache dtype");
  constexpr bool FP8 = DT == PKV_FP8_E4M3;
  using H = Fmt16<DT == PKV_F16>;                    // operand format of the products
  using x8 = typename H::x8;
  static_assert(HP == 1 || (HP == 2 && FP8), "two heads per wave: e4m3 caches");
  static_assert(D == 128 || (HP == 1 && !FP8), "head size 256: 16-bit caches");
  constexpr int kTile = Geo<D>::kTile;
  constexpr int kVPitch = Geo<D>::kVPitch;
  constexpr int kWaveLds = Geo<D>::kWaveLds;
  constexpr int kKSteps = D / 32;                    // k-steps of the logits product
  constexpr int kTT = kTile / 16;                    // 16-token blocks of a tile (2 or 1)
  constexpr int kNS = 4 * kTT;                       // logits of a lane per tile
  constexpr int kDB = D / 16;                        // 16-dim blocks of the output
  // probabilities as the B operand of the PV product: 8 values (32-token
  // tiles, 16 x 16 x 32 products) or 4 (16-token tiles, 16 x 16 x 16)
  using PB = std::conditional_t<kTT == 2, x8, typename H::x4>;
  // blocks a 32-token tile spans; a tile of larger blocks lies inside one
  // block (tiles start at multiples of 32 positions), at offset tbase % BS
  constexpr int kBlkPerTile = BS < kTile ? kTile / BS : 1;
  constexpr int kEB = FP8 ? 1 : 2;                   // bytes per cached element
  // bytes of one token's row as a wave reads it: HP adjacent kv heads
  constexpr int kRowBytes = HP * D * kEB;
  constexpr int kLanesPerRow = kRowBytes / 16;
  constexpr int kRowsPerLoad = 64 / kLanesPerRow;    // token rows per wave load
  constexpr int kLoads = kTile / kRowsPerLoad;       // loads per tile (K and V each)

  Item it;
  if (!resolve_item(a, a.seq_order ? load_uniform_i32(a.seq_order, zi) : zi, it)) return;
  // This workgroup covers partitions [part_first, part_end) of the row (one
  // "range"); ranges sit on the slowest grid axis so that the workgroups of
  // ranges a short sequence does not have dispatch last.
  const int rz = a.range_desc ? nz - 1 - bz : bz;
  const int part_first = rz * a.parts_per_wg;
  if (rz >= it.nranges) return;
  const int part_end = min(part_first + a.parts_per_wg, it.nparts);

  // The thread index passes through an empty asm: in a persistent grid that
  // runs this body and another per item, the lane-derived offsets are then
  // formed inside each body, not hoisted above the item loop and held in
  // registers across both bodies.
  int tid = threadIdx.x;
  __asm__ volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;     // MFMA column (query head) / A row (token or dim)
  const int kg = lane >> 4;    // k group / token row of a natural load
  const int group = a.num_heads / a.num_kv_heads;
  // HP == 2: bx is a pair of kv heads (head_chunks is 1), 2 bx and 2 bx + 1.
  // With one column per kv head (or pair), adjacent 256-byte rows swap
  // columns (column_head).
  const int kvh = HP == 2 ? 2 * column_head(bx, a.num_kv_heads / 2, kRowBytes)
                          : (a.head_chunks == 1 ? column_head(bx, a.num_kv_heads, kRowBytes)
                                                : bx / a.head_chunks);
  const int chunk = HP == 2 ? 0 : bx % a.head_chunks;
  const int h0 = kvh * group + chunk * 16;           // first query head of head hp: h0 + hp * group
  const int G = min(16, group - chunk * 16);

  const int pstart = it.base + part_first * it.P;
  const int pend = min(it.base + part_end * it.P, it.L_end);
  const int pbegin = it.L_begin;                 // first visible key (sliding window)

  // Q^T B operands: lane (kg, n) holds q[h0+n][(4j+kg)*8 .. +8] for k-step j.
  x8 qb[HP][kKSteps];
#pragma unroll
  for (int hp = 0; hp < HP; ++hp) {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((int64_t)it.row * a.num_heads + h0 + hp * group + n) * D;
#pragma unroll
    for (int j = 0; j < kKSteps; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (n < G) v = *reinterpret_cast<const u32x4*>(qrow + (4 * j + kg) * 8);
      qb[hp][j] = H::as_x8(v);
    }
  }

  f32x4 o[HP][kDB];
  float m[HP], lsum[HP], logit_scale[HP];
#pragma unroll
  for (int hp = 0; hp < HP; ++hp) {
#pragma unroll
    for (int jd = 0; jd < kDB; ++jd) o[hp][jd] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[hp] = kMinRef;
    lsum[hp] = 0.f;
    logit_scale[hp] = a.scale_log2;
    if constexpr (FP8) logit_scale[hp] *= a.k_scale[kvh + hp];
  }

  const int32_t* __restrict__ bt = a.block_tables + (int64_t)it.seq * a.max_blocks_per_seq;
  const char* __restrict__ kc = static_cast<const char*>(a.k_cache);
  const char* __restrict__ vc = static_cast<const char*>(a.v_cache);
  const uint32_t tok_stride = (uint32_t)a.num_kv_heads * D * kEB;   // bytes
  const uint32_t head_off = (uint32_t)kvh * D * kEB;
  const int64_t blk_stride = a.block_stride * kEB;
  // lane's place in a natural load: token row within the load, byte offset
  // in the row, and (fp8) which head's 128 bytes it holds
  const int lrow = lane / kLanesPerRow;
  const int lbyte = (lane % kLanesPerRow) * 16;
  const int lchunk = lane % kLanesPerRow;             // 16-byte chunk of the row it loads
  const int lhead = FP8 ? (lane % kLanesPerRow) / 8 : 0;
  const int64_t max_blk = a.num_blocks - 1;
  const int ntiles = (pend > pstart) ? (pend - pstart + kTile - 1) / kTile : 0;
  const int last_bi = (pend - 1) / BS;

  // the wave's LDS: HP areas of kWaveLds bytes, one per head
  char* wlds = s_lds + wave * HP * kWaveLds;

  // Block ids of one tile (wave uniform, scalar loads), fetched a step
  // early, as byte offsets of the tile's first token row in each block.
  auto fetch_ids = [&](int tile, int64_t* ids) {
    const int tbase = pstart + tile * kTile;
#pragma unroll
    for (int b = 0; b < kBlkPerTile; ++b) {
      const int bi = __builtin_amdgcn_readfirstlane(min(tbase / BS + b, last_bi));
      ids[b] = min((int64_t)max(load_uniform_i32(bt, bi), 0), max_blk) * blk_stride;
      if constexpr (BS > kTile) ids[b] += (int64_t)(tbase % BS) * tok_stride;
    }
  };

  // K (or V) loads of one tile: kLoads natural loads, each kRowsPerLoad
  // whole token rows (row kRowsPerLoad * i + lrow, 16 bytes at lbyte).  Each
  // such group of rows lies in one block (for blocks larger than the tile,
  // tok % BS = tok and ids[0] already points at the tile's first row).
  auto issue = [&](const char* cache, const int64_t* ids, u32x4* R) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int tok = kRowsPerLoad * i + lrow;
      const int64_t boff = ids[(kRowsPerLoad * i) / BS];
      const uint32_t lo = (uint32_t)(tok % BS) * tok_stride + head_off + lbyte;
      R[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cache + boff + lo));
    }
  };

  // Stage a tile's K rows, or its V rows (those of tokens past the end
  // become zeros), in the wave's LDS area (of the lane's head).
  auto stage_k = [&](const u32x4* K) {
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int tok = kRowsPerLoad * i + lrow;
      if constexpr (FP8) {
        // 16 codes = dims 16c .. 16c + 15 -> bfloat16 chunks 2c and 2c + 1
        const int c = lane & 7;
        char* klds = wlds + lhead * kWaveLds;
        u32x4 k0, k1;
        e4m3x16_to_bf16x16(K[i], k0, k1);
        *reinterpret_cast<u32x4*>(klds + ktile_off<D>(tok, 2 * c)) = k0;
        *reinterpret_cast<u32x4*>(klds + ktile_off<D>(tok, 2 * c + 1)) = k1;
      } else {
        *reinterpret_cast<u32x4*>(wlds + ktile_off<D>(tok, lchunk)) = K[i];
      }
    }
    __asm__ volatile("" ::: "memory");
  };
  auto stage_v = [&](int tile, const u32x4* V) {
    const int tbase = pstart + tile * kTile;
    const bool full = tbase + kTile <= pend && tbase >= pbegin;
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int tok = kRowsPerLoad * i + lrow;
      const bool dead = !full && (tbase + tok >= pend || tbase + tok < pbegin);
      if constexpr (FP8) {
        const int c = lane & 7;
        char* vlds = wlds + lhead * kWaveLds;
        u32x4 v0, v1;
        e4m3x16_to_bf16x16(V[i], v0, v1);
        if (dead) v0 = v1 = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(vlds + tok * kVPitch + c * 32) = v0;
        *reinterpret_cast<u32x4*>(vlds + tok * kVPitch + c * 32 + 16) = v1;
      } else {
        u32x4 v = V[i];
        if (dead) v = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(wlds + tok * kVPitch + lchunk * 16) = v;
      }
    }
    __asm__ volatile("" ::: "memory");
  };

  // Logits of head hp for a tile whose K rows are staged, and its online
  // softmax update: returns the probabilities (the B operand of the PV
  // product).
  auto logits = [&](int tile, int hp) {
    const int tbase = pstart + tile * kTile;
    const bool full = tbase + kTile <= pend && tbase >= pbegin;
    const char* klds = wlds + hp * kWaveLds;

    // logits S^T: A operand = K rows (token tt*16 + n, chunk 4j + kg)
    f32x4 sacc[kTT];
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      sacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kKSteps; ++j) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(klds + ktile_off<D>(tt * 16 + n, 4 * j + kg));
        sacc[tt] = H::mfma(H::as_x8(ka), qb[hp][j], sacc[tt]);
      }
    }
    // lane holds tokens tt*16 + 4kg + i of head column n
    float s[kNS];
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tbase + tt * 16 + 4 * kg + i;
        s[tt * 4 + i] = (full || (tok < pend && tok >= pbegin)) ? sacc[tt][i] * logit_scale[hp]
                                                                : -INFINITY;
      }
    // Probabilities against the current reference.  Some lane's sum can
    // exceed 2^slack only if its column's max outgrew the reference by more
    // than the slack (or several of its probabilities are large); then, and
    // only then, the wave takes the full step: the tile's column maxima, the
    // raised references with the rescale, and the probabilities again.  The
    // result is the same as always taking it.
    PB pb;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < kNS; ++e) {
      const float p = fast_exp2(s[e] - m[hp]);
      psum += p;
      pb[e] = (typename H::elem)p;
    }
    if (__builtin_amdgcn_ballot_w64(!(psum <= kSlackSum))) {
      float mx = s[0];
#pragma unroll
      for (int e = 1; e < kNS; ++e) mx = fmaxf(mx, s[e]);
      mx = xmax16_32(mx);                            // the same on the column's 4 lanes
      if (mx > m[hp] + kRescaleSlack) {
        const float alpha = fast_exp2(m[hp] - mx);
        lsum[hp] *= alpha;
#pragma unroll
        for (int jd = 0; jd < kDB; ++jd) o[hp][jd] *= alpha;
        m[hp] = mx;
      }
      psum = 0.f;
#pragma unroll
      for (int e = 0; e < kNS; ++e) {
        const float p = fast_exp2(s[e] - m[hp]);
        psum += p;
        pb[e] = (typename H::elem)p;
      }
    }
    lsum[hp] += psum;
    __asm__ volatile("" ::: "memory");
    return pb;
  };

  // O^T += V^T P^T for head hp of a tile whose V rows are staged, one 16-dim
  // tile at a time; the transposed reads give lane (kg, n) V[4kg + jj][16jd + n]
  // and V[16 + 4kg + jj][16jd + n].
  auto pv = [&](const PB pb, int hp) {
    {
      const int jj = n >> 2, q4 = n & 3;
      const char* r0 = wlds + hp * kWaveLds + (4 * kg + jj) * kVPitch + q4 * 8;
      const char* r1 = r0 + 16 * kVPitch;
#pragma unroll
      for (int jd = 0; jd < kDB; ++jd) {
        i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(r0 + jd * 32));
        if constexpr (kTT == 2) {
          i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(r1 + jd * 32));
          const x8 va = __builtin_bit_cast(x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[hp][jd] = H::mfma(va, pb, o[hp][jd]);
        } else {
          // 16-token tiles: the first transposed read is the whole A operand
          o[hp][jd] = H::mfma16(__builtin_bit_cast(typename H::x4, lo), pb, o[hp][jd]);
        }
      }
    }
    __asm__ volatile("" ::: "memory");
  };

  // The tile stream of this wave.  Tile t's K rows are waited for and
  // copied into LDS, the next tile's K loads are issued into the same
  // registers, the logits are computed; then the same for the V rows and the
  // PV product.  Loads stay in flight while the wave computes, and block ids
  // run one tile further ahead.  Either wave w owns partition w of the range
  // (long rows: waves never wait for each other), or the waves take the
  // range's tiles round-robin (short rows: every wave gets work).
  const int tpp = it.P / kTile;                      // tiles per partition (split rows)
  int tile, tstep, tend;
  if (a.wave_per_part && it.nparts > 1 && part_end - part_first == kWaves) {
    tile = wave * tpp;
    tend = min(ntiles, (wave + 1) * tpp);
    tstep = 1;
  } else {
    tile = wave;
    tend = ntiles;
    tstep = kWaves;
  }
  u32x4 kr[kLoads], vr[kLoads];
  int64_t ids[kBlkPerTile];
  if (tile < tend) {
    fetch_ids(tile, ids);
    issue(kc, ids, kr);
    issue(vc, ids, vr);
    if (tile + tstep < tend) fetch_ids(tile + tstep, ids);
  }
  while (tile < tend) {
    const int nt = tile + tstep;
    stage_k(kr);
    if (nt < tend) issue(kc, ids, kr);
    PB pb[HP];
#pragma unroll
    for (int hp = 0; hp < HP; ++hp) pb[hp] = logits(tile, hp);
    stage_v(tile, vr);
    if (nt < tend) {
      issue(vc, ids, vr);
      if (nt + tstep < tend) fetch_ids(nt + tstep, ids);
    }
#pragma unroll
    for (int hp = 0; hp < HP; ++hp) pv(pb[hp], hp);
    tile = nt;
  }

  // Merge the 4 waves (log-sum-exp rule) per head and write the row, or this
  // range's partial result.  Each wave stages its state inside its own LDS
  // areas.
#pragma unroll
  for (int hp = 0; hp < HP; ++hp) {
    lsum[hp] = xsum16_32(lsum[hp]);
    float* so = reinterpret_cast<float*>(wlds + hp * kWaveLds);   // [16 heads][D]
#pragma unroll
    for (int jd = 0; jd < kDB; ++jd)
      *reinterpret_cast<f32x4*>(so + n * D + 16 * jd + 4 * kg) = o[hp][jd];
    if (kg == 0) {
      s_m[wave][hp * 16 + n] = m[hp];
      s_l[wave][hp * 16 + n] = lsum[hp];
    }
  }
  __syncthreads();
  const int range = rz;
  for (int idx = tid; idx < HP * G * D; idx += kThreads) {
    const int hp = idx / (G * D);
    const int h = (idx / D) % G;
    const int d = idx % D;
    float M = s_m[0][hp * 16 + h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][hp * 16 + h]);
    const float Mref = (M == -INFINITY) ? 0.f : M;
    float O = 0.f, Ls = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(s_m[w][hp * 16 + h] - Mref);
      O = fmaf(reinterpret_cast<const float*>(s_lds + (w * HP + hp) * kWaveLds)[h * D + d], f, O);
      Ls = fmaf(s_l[w][hp * 16 + h], f, Ls);
    }
    const int head = h0 + hp * group + h;
    float out_scale = 1.f;
    if constexpr (FP8) out_scale = a.v_scale[kvh + hp];
    if (it.nranges == 1) {
      const float v = Ls > 0.f ? O / Ls * out_scale : 0.f;
      static_cast<uint16_t*>(a.out)[((int64_t)it.row * a.num_heads + head) * D + d] =
          static_cast<uint16_t>(H::rne(v));
      if (d == 0 && a.lse_out)
        a.lse_out[(int64_t)it.row * a.num_heads + head] =
            Ls > 0.f ? (M + acc_log2(Ls)) * kLn2 : -INFINITY;
    } else {
      const int64_t widx = ((int64_t)range * a.num_heads + head) * a.num_seqs + it.seq;
      a.ws_o[widx * D + d] = Ls > 0.f ? O / Ls * out_scale : 0.f;
      if (d == 0) a.ws_lse[widx] = Ls > 0.f ? M + acc_log2(Ls) : -INFINITY;
    }
  }
}

}  // namespace dec
}  // namespace pkv
