// verify_attn.hip -- tree-verify attention in absorbed MLA form for gfx950.
//
// Computes what "The Architecture of a Thousand-Parameter Decision ..." ("What
// to Build New", item 2) asks of the tree-verify kernel, in the absorbed form
// of "The Milestone Message ..." ("MLA"): every tree node of every request
// attends over the request's latent prefix (always visible) and over the tree
// entries its visibility bitset allows (ancestors and itself, "Architectural
// Abstraction").  Keys are the 576-wide [c_kv | k_pe] rows, values the 512-wide
// c_kv rows, and the output stays in latent space.
//
// Mapping to CDNA4:
//  * Rows of a request are (node, head) pairs, row = i*H + h, so one request is
//    an M = Q*H by 576 query matrix against its shared keys.  A row tile is 128
//    rows; keys stream in tiles of 32, loaded global -> LDS directly (16 bytes
//    per lane, no register staging) one tile ahead into a ring of three stages,
//    with the pool slot ids of each tile fetched two tiles ahead into a small
//    LDS ring.  All products are 32x32x16 bf16 MFMAs (fp32 inputs: 32x32x2
//    f32) with fp32 accumulation.
//  * Three forms of the same computation:
//     - wide (bf16 512+64, the default): four waves per workgroup, one per
//       SIMD, each owning 32 rows with their whole query (36 operand
//       registers) and whole output (the 256 accumulator registers), so both
//       contractions and the softmax of a row stay inside one wave; the
//       softmax of tile t runs while the value product of tile t-1 does;
//     - narrow (bf16 512+64, very few row tiles, as at batch 1): four
//       workgroups of 32 rows share each key range; inside one, the four waves
//       split the score contraction and the output columns, and sum their
//       partial scores in LDS;
//     - paired-wave (64-wide latent rows, bf16 and fp32): two waves per 32
//       rows, each with half of the query dimensions and half of the output
//       columns, exchanging partial scores through LDS.
//    Scores are computed transposed, S^T = K Q^T, so that in the accumulator
//    layout each lane owns one row and 16 of the 32 keys -- the B operand
//    layout of O^T = V^T P^T -- and probabilities never leave registers.  The
//    V^T operand comes from the same key-major tile through the transposing
//    LDS read (ds_read_b64_tr_b16).
//  * Softmax in the exp2 domain with fp32 statistics.  The wide and narrow
//    forms use a fixed reference per row (its first tile's max) and run a
//    range again from its start, with the largest score seen as reference, in
//    the rare case that a later score would overflow; the paired-wave form
//    moves its reference when a row's max grows by more than 2^8.  The
//    probabilities are rounded to bf16 for the value product; when a tile
//    holds a key whose weight is a sizeable share of its row's running sum,
//    the bf16 rounding residual goes through a second MFMA against the same
//    value operand, which brings the value product to ~2^-16 relative
//    accuracy.
//  * The mask: prefix keys are always visible; a tree key k is visible when bit
//    k of the row's node bitset is set; keys beyond the request or with a slot
//    id outside the pool are invisible (their tile rows hold pool row 0, which
//    a zero probability then ignores).
//  * Work split (attn_split.h): the (request, row tile, key tile) space is cut
//    into equal contiguous ranges, one per workgroup of a grid sized to the
//    chip, so ragged prefixes stay balanced; uniform batches with at least one
//    row tile per workgroup take an aligned split instead (whole row tiles
//    first, then the leftover row tiles cut evenly).  Logical workgroup ids are
//    remapped so that consecutive ranges land on the same XCD and share its L2.
//    A row tile whose key range is cut writes normalised partial outputs plus
//    their log-sum-exp to the workspace, and a merge kernel combines them.
//  * Output and partial rows are stored at device scope (write-through past the
//    XCD's L2), so the kernel's end has no dirty lines to write back before the
//    merge may start.
#include <stdlib.h>

#include <type_traits>

#include "ddt_internal.h"

namespace ddt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4_lds_t __attribute__((__vector_size__(4 * sizeof(__bf16))));
#define DDT_LDS __attribute__((address_space(3)))

constexpr int kSplit = 2;                // waves sharing one 32-row block
constexpr int kWaves = 4 * kSplit;
constexpr int kThreads = kWaves * kWave;
// Slot-id ring: tiles kb-1 .. kb+2.  A wave publishes the slot ids of tile
// kb+2 during step kb, while a slower wave of the same step may still mask
// tile kb-1 with that tile's validity bits, so four entries are live.
constexpr int kRing = 4;
constexpr int kStages = 3;               // key-tile stages in LDS (tiles kb-1 .. kb+1)
constexpr int kMergeThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// A tile takes the residual pass when some key's probability exceeds this share
// of its row's running sum (an upper bound on the key's final weight).  A key
// below it carries at most a sixteenth of the row's weight, so leaving its
// bf16 rounding (round to nearest: relative 2^-8 at most) uncorrected moves the
// output by at most 2^-12 times the largest value entry.
constexpr float kHeavyShare = 1.0f / 16.0f;
// Reference-max slack of the online softmax, in log2 units.
constexpr float kRescaleLog2 = 8.0f;

// T is the storage type: uint16_t for bf16, float for fp32.
template <typename T, int DL, int DR>
struct Geo {
  static constexpr bool kBF16 = std::is_same<T, uint16_t>::value;
  static constexpr int kElt = sizeof(T);
  static constexpr int kDK = DL + DR;
  static constexpr int kPerChunk = 16 / kElt;               // elements per 16-byte chunk
  static constexpr int kLatChunks = DL / kPerChunk;         // 16-byte chunks of a latent row
  static constexpr int kPeChunks = DR / kPerChunk;          // ... of a rope row
  // Latent region.  A 64-chunk row (bf16, 512 wide) is one load instruction
  // and sits at a 1 KiB pitch with its 16-byte chunks permuted per key (see
  // swz()), which keeps both the operand reads of QK^T and the transposing
  // reads of PV free of bank conflicts; smaller rows pack several keys per
  // instruction, unpermuted.
  static constexpr bool kSwz = kLatChunks == kWave;
  static constexpr int kKeysPerInstr = kLatChunks >= kWave ? 1 : kWave / kLatChunks;
  static constexpr int kLatPitchB = kLatChunks * 16;
  static constexpr int kLatPitch = kLatPitchB / kElt;       // in elements
  static constexpr int kLatInstr = kTileKeys / kKeysPerInstr * (kLatChunks >= kWave ? kLatChunks / kWave : 1);
  // Rope region: keys back to back; 8-chunk rows are XOR-swizzled by key.
  static constexpr int kPeInstr = (kTileKeys * kPeChunks + kWave - 1) / kWave;
  static constexpr int kLatBytes = kTileKeys * kLatPitchB;
  static constexpr int kStageBytes = kLatBytes + kPeInstr * kWave * 16;
  static constexpr int kStageElems = kStageBytes / kElt;
  static constexpr int kInstr = kLatInstr + kPeInstr;       // load instructions per tile
  static_assert(kLatChunks <= kWave || kLatChunks == kWave, "latent row size");
  static constexpr int kKStep = kBF16 ? 16 : 2;             // contraction depth of one MFMA
  static constexpr int kNK = kDK / kKStep;                  // MFMAs per 32x32 score block
  static constexpr int kNK0 = (kNK + kSplit - 1) / kSplit;  // ... done by each wave of a group
  static constexpr int kNCB = DL / 32;                      // 32-wide output column blocks
  static constexpr int kNCBh = kNCB / kSplit;               // ... owned by each wave of a group
  static constexpr int kIssuePerWave = (kInstr + kWaves - 1) / kWaves;
  static_assert(kNCB % kSplit == 0, "column split");
  static_assert(DL % 32 == 0 && DR % 16 == 0, "head dims");
  static_assert(kDK % kKStep == 0, "contraction depth");
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Eight probabilities as a bf16x8 operand (round to nearest even, v_cvt_pk_bf16_f32);
// with kResidual, the rounding residuals p - bf16(p) instead, which are exact
// in fp32 and rounded to bf16 once more.
template <bool kResidual>
__device__ __forceinline__ bf16x8_t pack_p(const float* p) {
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x2_t v = {p[2 * k], p[2 * k + 1]};
    bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    if constexpr (kResidual) h = __builtin_convertvector(v - __builtin_convertvector(h, f32x2_t), bf16x2_t);
    w[k] = __builtin_bit_cast(uint32_t, h);
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
}


// Wave-uniform values read from LDS or derived from them are moved to scalar
// registers so they do not occupy vector registers.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long long uni(long long v) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(v & 0xFFFFFFFFll));
  const int hi = __builtin_amdgcn_readfirstlane((int)(v >> 32));
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
// The value lane `l` holds (l uniform).
__device__ __forceinline__ long long lane_value(long long v, int l) {
  const int lo = __builtin_amdgcn_readlane((int)(v & 0xFFFFFFFFll), l);
  const int hi = __builtin_amdgcn_readlane((int)(v >> 32), l);
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// The split of a launch: mode (split_mode, -1 for one stream) and the start
// cost c of a row tile in the stream.
struct SplitMode {
  long long mode;
  int c;
};

// One DPP step of a wave scan: the value of the lane CTRL selects, 0 where it
// selects none (rows outside ROW_MASK, lanes shifted in at a row's start).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_take(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ long long dpp_take(long long v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = (uint32_t)dpp_take<CTRL, ROW_MASK>((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)dpp_take<CTRL, ROW_MASK>((int)(uint32_t)(u >> 32));
  return (long long)(((uint64_t)hi << 32) | lo);
}

// Inclusive sum over lanes 0..lane of a wavefront: shifts by 1, 2, 4, 8
// inside each 16-lane row, then row 0's total into row 1 and row 2's into row
// 3 (row_bcast:15), then the total of rows 0-1 into rows 2 and 3
// (row_bcast:31).
template <typename V>
__device__ __forceinline__ V wave_inclusive_sum(V v) {
  v += dpp_take<0x111, 0xF>(v);  // row_shr:1
  v += dpp_take<0x112, 0xF>(v);  // row_shr:2
  v += dpp_take<0x114, 0xF>(v);  // row_shr:4
  v += dpp_take<0x118, 0xF>(v);  // row_shr:8
  v += dpp_take<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_take<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// Exclusive stream prefix over requests into s_pref[0..B] (each row tile with
// work is a segment of nkb + c positions) and (when s_req is given) each
// request's clamped prefix length and tree size into s_req[0..B); called by
// all threads of a workgroup, computed by its first wave and published with
// one barrier; s_wsum holds at least 2 values.  Request b sits in lane b % 64
// of row b / 64; a row is one wave scan, so batches up to 64 take one.  The
// split mode applies to a launch of 2G workgroups (split2); the start cost c
// follows from the split mode and the request sizes.
template <int kBlock>
__device__ SplitMode work_prefix(long long* s_pref, long long* s_wsum, int2* s_req,
                                 const int32_t* prefix_len, const int32_t* n_nodes, int B, int Q,
                                 int H, int max_kv, int RT, long long G, bool split2) {
  static_assert(kBlock >= kWave, "one full wavefront computes the prefix");
  constexpr int kRows = kMaxBatch / kWave;
  const int t = threadIdx.x;
  if (t < kWave) {
    const ReqInfo r0 = req_info(prefix_len, n_nodes, 0, Q, H, max_kv, RT);
    long long ew[kRows];  // work of the requests before this one
    long long ev[kRows];  // row tiles with work before this one
    long long wtot = 0, vtot = 0;
    bool differs = false;
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      ew[k] = 0;
      ev[k] = 0;
      if (k * kWave < B) {
        const int b = k * kWave + t;
        long long w = 0, v = 0;
        if (b < B) {
          const ReqInfo r = req_info(prefix_len, n_nodes, b, Q, H, max_kv, RT);
          w = (long long)r.vt * r.nkb;
          v = r.vt;
          if (r.vt != r0.vt || r.nkb != r0.nkb) differs = true;
          if (s_req) s_req[b] = make_int2(r.L, r.nb);
        }
        const long long iw = wave_inclusive_sum(w);
        const long long iv = wave_inclusive_sum(v);
        ew[k] = wtot + iw - w;
        ev[k] = vtot + iv - v;
        wtot += lane_value(iw, kWave - 1);
        vtot += lane_value(iv, kWave - 1);
      }
    }
    const bool same = __ballot(differs) == 0;
    SplitMode sp;
    sp.mode = split2 ? split_mode(same, r0.vt, B, G) : -1;
    sp.c = unit_cost(sp.mode, same, vtot, G);
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const int b = k * kWave + t;
      if (b < B) s_pref[b] = ew[k] + sp.c * ev[k];
    }
    if (t == 0) {
      s_pref[B] = wtot + sp.c * vtot;
      s_wsum[0] = sp.mode;
      s_wsum[1] = sp.c;
    }
  }
  __syncthreads();
  SplitMode sp;
  sp.mode = s_wsum[0];
  sp.c = (int)s_wsum[1];
  return sp;
}

template <typename T, int DL, int DR>
struct Smem {
  using G = Geo<T, DL, DR>;
  alignas(1024) unsigned char stage[kStages][G::kStageBytes];
  alignas(16) int32_t slot[kRing][kTileKeys];  // pool slot of each key of a tile (0 when invalid)
  uint32_t valid[kRing];            // bit m: key m of the tile is in range with a valid slot
  float4 xs[kWaves][2][kWave];      // partial scores of the partner's keys
  float4 xp[kWaves][G::kBF16 ? 1 : 2][kWave];  // probabilities of own keys (bf16: packed)
  uint4 xr[kWaves][kWave];          // bf16 rounding residuals of own keys
  float xm[kWaves][kWave];          // row max over own keys
  float xl[kWaves][kWave];          // row sum over own keys
  int xflag[kWaves];                // posted sequence numbers
  uint32_t xheavy[kWaves];          // residuals posted with the latest probabilities
  uint64_t visrow[kRowsPerWG][2];   // visibility bitset of each row's tree node
  long long pref[kMaxBatch + 1];
  int2 req[kMaxBatch];  // per request: clamped prefix length, tree size
  long long wsum[2 * kWaves];
};

// Raw pool slot id of key `j` of the request (-1 past the request); its range
// is checked when it is published, so the load's latency is not waited for
// where it is issued.
__device__ __forceinline__ int32_t fetch_slot(const int32_t* __restrict__ slots_b, int j,
                                              int nkeys) {
  return j < nkeys ? slots_b[j] : -1;
}

// Latent chunk permutation of the 1 KiB-pitch layout: logical 16-byte chunk c
// of key row r is stored at chunk c ^ swz(r), swz(r) = A[r & 3] ^ ((r >> 2) & 3)
// with A = {0, 4, 10, 14}.  Over each aligned group of 16 keys swz takes 16
// distinct values, and their low 3 bits differ within each aligned group of 8
// keys (operand reads of one chunk by 8 or 16 keys cover distinct banks); bits
// 2..3 differ within each aligned group of 4 keys (transposing reads of 4 keys
// x 64 bytes cover all banks).
__device__ __forceinline__ int swz_a(int r) { return (0xEA40 >> (4 * (r & 3))) & 15; }
__device__ __forceinline__ int swz(int r) { return swz_a(r) ^ ((r >> 2) & 3); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const DDT_LDS void*)p;
}

// Physical chunk of logical rope chunk c of key `key` (8-chunk rows only).
template <int kPeChunks>
__device__ __forceinline__ int pe_swz(int c, int key) {
  if constexpr (kPeChunks == 8) return c ^ (key & 7);
  else return c;
}

// A 16-byte store at device scope (sc1): it writes through this XCD's L2, so
// the row leaves no dirty line behind for the release at the kernel's end,
// which otherwise writes back every workgroup's output after the last one
// finishes.  A vector store with no result register.
__device__ __forceinline__ void store_through(float* d, const float4 v) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const v4f x = {v.x, v.y, v.z, v.w};
  __asm__ __volatile__("global_store_dwordx4 %0, %1, off sc1" : : "v"(d), "v"(x) : "memory");
}

// Direct global -> LDS load of 16 bytes per lane: lane l's bytes land at LDS
// address lds + 16*l.  Issued as inline assembly: the compiler's wait-count
// pass would otherwise make every later LDS read wait for these loads (it
// cannot tell that they target the other stage), which would serialise each
// tile behind the next tile's memory latency.  The kernel waits for them
// itself (s_waitcnt vmcnt(0) before the barrier that publishes a stage).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  __asm__ __volatile__("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                       :
                       : "v"(src), "s"(lds)
                       : "memory", "m0");
}
#pragma clang diagnostic pop

// Enqueue the direct global->LDS loads of one key tile.  With 64-chunk latent
// rows, wave w loads latent rows of keys kLatInstr/kWaves*w.. (one row per
// instruction, slot read as a scalar) and, for w < kPeInstr, one instruction of
// 8 keys x 8 rope chunks; otherwise instructions are dealt round-robin.
// Invalid keys carry slot 0 (pool row 0), which the mask ignores.
template <typename T, int DL, int DR>
__device__ __forceinline__ void issue_tile(unsigned char* stage, const int32_t* ring_slots,
                                           const T* __restrict__ c_kv,
                                           const T* __restrict__ k_pe, int wave, int lane) {
  using G = Geo<T, DL, DR>;
  if constexpr (G::kLatChunks == kWave && G::kPeChunks == 8 && G::kLatInstr % kWaves == 0) {
    constexpr int kPerWave = G::kLatInstr / kWaves;
    static_assert(kPerWave == 4, "one 16-byte read of slot ids per wave");
    // This wave's four latent keys in one LDS read, and (waves < kPeInstr) the
    // rope key of this lane, before waiting on either.
    const int4 sl = *reinterpret_cast<const int4*>(ring_slots + wave * kPerWave);
    const int pe_key = wave * 8 + (lane >> 3);
    const int pe_row = wave < G::kPeInstr ? ring_slots[pe_key] : 0;
    const int rows[4] = {sl.x, sl.y, sl.z, sl.w};
#pragma unroll
    for (int it = 0; it < kPerWave; ++it) {
      const int key = wave * kPerWave + it;
      const long long row = uni(rows[it]);
      // Lane l fills physical chunk l, i.e. logical chunk l ^ swz(key).
      dma16(static_cast<const void*>(c_kv + row * DL + (lane ^ swz(key)) * G::kPerChunk),
            lds_addr(stage + key * G::kLatPitchB));
    }
    if (wave < G::kPeInstr) {
      // 8 keys x 8 chunks; key & 7 == lane / 8, so the swizzled chunk depends
      // on the lane only.
      const T* src = k_pe + (long long)pe_row * DR + (((lane & 7) ^ (lane >> 3)) * G::kPerChunk);
      dma16(static_cast<const void*>(src), lds_addr(stage + G::kLatBytes + wave * kWave * 16));
    }
  } else {
#pragma unroll
    for (int it = 0; it < G::kIssuePerWave; ++it) {
      const int r = wave + it * kWaves;
      if (r >= G::kInstr) break;
      if (r < G::kLatInstr) {
        int key, ch;
        unsigned char* dst;
        if constexpr (G::kLatChunks >= kWave) {
          constexpr int kPerKey = G::kLatChunks / kWave;
          key = r / kPerKey;
          ch = (r % kPerKey) * kWave + lane;
          dst = stage + key * G::kLatPitchB + (r % kPerKey) * kWave * 16;
        } else {
          key = r * G::kKeysPerInstr + lane / G::kLatChunks;
          ch = lane % G::kLatChunks;
          dst = stage + r * kWave * 16;
        }
        const long long row = ring_slots[key];
        dma16(static_cast<const void*>(c_kv + row * DL + ch * G::kPerChunk), lds_addr(dst));
      } else {
        const int rp = r - G::kLatInstr;
        const int s = rp * kWave + lane;  // rope chunk slot
        const int key = s / G::kPeChunks;
        const int p = s % G::kPeChunks;
        const T* src = k_pe;              // slack lanes past the tile
        if (key < kTileKeys) {
          const long long row = ring_slots[key];
          src = k_pe + row * DR + pe_swz<G::kPeChunks>(p, key) * G::kPerChunk;
        }
        dma16(static_cast<const void*>(src), lds_addr((stage + G::kLatBytes + rp * kWave * 16)));
      }
    }
  }
}

// Two transposing reads give the 8-key A operand of one value-product MFMA:
// keys k0..k0+3 and k0+8..k0+11 of column `col` for this lane.
__device__ __forceinline__ bf16x8_t read_vt(const uint16_t* kt, int pitch, int k0, int col0,
                                            int lane) {
  const int j = lane & 15;
  const uint16_t* pa = kt + (k0 + (j >> 2)) * pitch + col0 + 4 * (j & 3);
  const uint16_t* pb = pa + 8 * pitch;
  const bf16x4_lds_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((DDT_LDS bf16x4_lds_t*)pa);
  const bf16x4_lds_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((DDT_LDS bf16x4_lds_t*)pb);
  const uint2 ulo = __builtin_bit_cast(uint2, lo);
  const uint2 uhi = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8_t, make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
}

// Transposing reads of the permuted 1 KiB-pitch latent rows.  Lane (j = l % 16,
// q = l / 16, g = l / 32) reads key row kbase + j/4 at logical column
// 32*cb + 16*(q%2) + 4*(j%4), i.e. logical chunk 4*cb + x (x = 2*(q%2) + (j%4)/2),
// half-chunk j%2.  For kbase = 4g + 8t + 16*k1 the row's swz is f0 = A[j/4] ^ g
// (t = 0) or f0 ^ 2 (t = 1), so with cb = 4h + c the byte address is
// (P_t ^ 64c) + 256h + 8192t + 16384*k1, P_t holding the row, the low chunk
// bits and the lane's half-chunk.
struct VtAddr {
  uint32_t p0, p1;
  __device__ __forceinline__ VtAddr(uint32_t tile, int lane) {
    const int j = lane & 15, q = lane >> 4, g = lane >> 5;
    const int x = 2 * (q & 1) + ((j & 3) >> 1);
    const int f0 = swz_a(j >> 2) ^ g, f1 = f0 ^ 2;
    const uint32_t rb = tile + (4 * g + (j >> 2)) * 1024 + 8 * (j & 1);
    p0 = rb + 16 * ((x ^ f0) & 3) + 64 * (f0 >> 2);
    p1 = rb + 16 * ((x ^ f1) & 3) + 64 * (f1 >> 2);
  }
  __device__ __forceinline__ bf16x8_t read(int cb, int k1) const {
    const uint32_t c = 64 * (cb & 3), h = 256 * (cb >> 2) + 16384 * k1;
    const bf16x4_lds_t lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((DDT_LDS bf16x4_lds_t*)(uintptr_t)((p0 ^ c) + h));
    const bf16x4_lds_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (DDT_LDS bf16x4_lds_t*)(uintptr_t)((p1 ^ c) + h + 8192));
    const uint2 ulo = __builtin_bit_cast(uint2, lo);
    const uint2 uhi = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8_t, make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
  }
};

// Lanes 0..31 of wave 0 store the slot ids of one tile (a key past the request
// or with a slot id outside the pool -> pool row 0) and its validity bitmask.
__device__ __forceinline__ void publish_slots(int32_t* ring, uint32_t* valid, int32_t raw,
                                              int64_t num_slots, int key) {
  const int32_t slot = (raw >= 0 && (int64_t)raw < num_slots) ? raw : -1;
  ring[key] = slot < 0 ? 0 : slot;
  const uint64_t ok = __ballot(slot >= 0);
  if (key == 0) *valid = (uint32_t)ok;
}

// Visibility of the 32 keys of a tile for one row: bit m is set when key m is a
// prefix key (tree index jb + m < 0) or the row's bitset has bit jb + m.
// jb > -32 (the tile reaches the tree part) and jb < 128.
__device__ __forceinline__ uint32_t tree_window(uint64_t v0, uint64_t v1, int jb) {
  if (jb < 0) {
    const int pc = -jb;  // 1..31 prefix keys at the start of the tile
    return ((1u << pc) - 1u) | (uint32_t)(v0 << pc);
  }
  if (jb == 0) return (uint32_t)v0;
  if (jb < 64) return (uint32_t)((v0 >> jb) | (v1 << (64 - jb)));
  return (uint32_t)(v1 >> (jb - 64));
}

// Everything one workgroup needs to process one row tile over a key range.
struct Unit {
  int b, rt, kb0, kb1, nkeys;
  ReqInfo ri;
  bool complete;
  long long slot;  // workspace slot when the key range is cut
};

struct Args {
  const void* q_lat;
  const void* q_pe;
  const void* c_kv;
  const void* k_pe;
  int64_t num_slots;
  const int32_t* req_to_slot;
  int max_kv;
  const uint64_t* vis;
  int Q, H;
  float sl2;  // softmax scale in log2 units
  float* out;
  float* lse;
  float* ws_o;
  float* ws_lse;
  int spin_limit;  // polls of a pair wait before it gives up (pair kernel)
};

// Sums / maxima of a value over lanes l and l ^ 32 (the two lanes of one row),
// bit-identical in both lanes.
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Pair synchronisation through LDS.  A wave posts an increasing sequence number
// once its LDS writes have completed; its partner waits until it sees that
// number.  Both waves of a pair take the same path, so they post the same
// sequence.  The wait is bounded so that it always ends; a wait that gives up
// marks the wave as stalled, and a stalled wave writes NaN for its rows (and
// their log-sum-exp), so the give-up can never pass as a result.
constexpr int kSpinLimit = 1 << 16;  // polls of ~100 cycles: milliseconds, far beyond a tile

__device__ __forceinline__ void pair_post(int* flag, int seq) {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
  __asm__ __volatile__("" ::: "memory");
  __hip_atomic_store(flag, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void pair_wait(int* flag, int seq, int limit, bool& stalled) {
  bool seen = false;
  for (int i = 0; i < limit; ++i) {
    if (uni(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) >= seq) {
      seen = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  stalled = stalled || !seen;
  __asm__ __volatile__("" ::: "memory");
}

// One row tile over key tiles [kb0, kb1) by the waves of share HALF (compile
// time, so every LDS operand address is one base register plus an immediate).
// The two waves of a pair split the work of each tile three ways:
//   QK^T  over their half of the 576 contraction dimensions (partial scores of
//         all 32 keys), then exchange the partial scores of the partner's keys;
//   softmax over their own 16 keys (HALF 0: keys 0..15, HALF 1: keys 16..31),
//         then exchange the bf16 probabilities of those keys and the row max;
//   PV    over their half of the 512 output columns with all 32 keys.
// The reference max of each row is the same in both waves: it only moves on
// the pair's combined tile max.  Probabilities are computed against the
// current reference before the maxima are exchanged; in the rare tiles where
// the reference moves, both waves recompute and exchange them again.
// Iteration t issues the loads of tile t+1, then runs PV of tile t-1 and QK
// and softmax of tile t, so tiles t-1 and t are read while t+1 loads: the key
// tiles rotate through three LDS stages (stage of tile t = t mod 3).
template <typename T, int DL, int DR, int HALF>
__device__ __forceinline__ void run_unit(Smem<T, DL, DR>& sm, const Args& a, const Unit& u,
                                         int& seq) {
  using G = Geo<T, DL, DR>;
  constexpr int kStep0 = HALF * G::kNK0;
  constexpr int kStep1 = (HALF + 1) * G::kNK0 < G::kNK ? (HALF + 1) * G::kNK0 : G::kNK;
  constexpr int kCb0 = HALF * G::kNCBh;
  constexpr int kOwn = 8 * HALF;    // first score register of this wave's keys
  constexpr int kMate = 8 - kOwn;   // first score register of the partner's keys
  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6);  // wave-uniform: keep it (and what derives from it) scalar
  const int mate = wave ^ 1;
  // An opaque copy of the lane id: nothing lane-derived is hoisted out of the
  // unit loop (values held across it would not fit the register budget).
  int lane = tid;
  __asm__ __volatile__("" : "+v"(lane));
  lane &= 63;
  const int rb = wave / kSplit;
  const int n = lane & 31;
  const int g = lane >> 5;
  const int W = (a.Q + 63) >> 6;
  const long long QH = (long long)a.Q * a.H;
  const T* q_lat = static_cast<const T*>(a.q_lat);
  const T* q_pe = static_cast<const T*>(a.q_pe);
  const T* c_kv = static_cast<const T*>(a.c_kv);
  const T* k_pe = static_cast<const T*>(a.k_pe);
  const int32_t* slots_b = a.req_to_slot + (long long)u.b * a.max_kv;

  // Slot ids of the first two tiles are requested before anything else: the
  // first tile's loads depend on them, the query and visibility rows do not.
  int32_t raw0 = -1, raw1 = -1;
  if (tid < kTileKeys) {
    raw0 = fetch_slot(slots_b, u.kb0 * kTileKeys + tid, u.nkeys);
    if (u.kb0 + 1 < u.kb1) raw1 = fetch_slot(slots_b, (u.kb0 + 1) * kTileKeys + tid, u.nkeys);
  }

  // This lane's row.
  const long long r_loc = (long long)u.rt * kRowsPerWG + rb * 32 + n;  // row in request
  int heads = a.H;  // opaque: the division's reciprocal is formed per unit, not held
  __asm__ __volatile__("" : "+s"(heads));
  const int node = (int)(r_loc / heads);
  const bool row_exists = r_loc < QH;
  const bool row_live = row_exists && node < u.ri.nb;
  const bool wave_live = __ballot(row_live) != 0;  // the same in both waves of the pair
  const long long grow = (long long)u.b * QH + r_loc;

  // Visibility row of this lane's node.
  uint64_t vis0 = 0, vis1 = 0;
  if (HALF == 0 && g == 0 && row_live) {
    const uint64_t* vr = a.vis + ((long long)u.b * a.Q + node) * W;
    vis0 = vr[0];
    if (W > 1) vis1 = vr[1];
  }

  // Query operand: B slots of this lane's row for contraction steps of HALF.
  using QV = typename std::conditional<G::kBF16, bf16x8_t, float>::type;
  QV q[kStep1 - kStep0];
  f32x16_t o[G::kNCBh];
#pragma unroll
  for (int cb = 0; cb < G::kNCBh; ++cb) o[cb] = f32x16_t{};
  // m_run: the row's reference max (log2 units), identical in both waves of the
  // pair; l_run: this lane's share of the row sum (own keys, its 8 of them).
  float m_run = -INFINITY, l_run = 0.0f;
  bool stalled = false;  // a pair wait of this wave gave up

  // Prologue: publish the slot ids and visibility rows, then issue the first
  // tile's loads and after them the query loads (both land together).
  if (tid < kTileKeys) {
    publish_slots(sm.slot[u.kb0 % kRing], &sm.valid[u.kb0 % kRing], raw0, a.num_slots, tid);
    if (u.kb0 + 1 < u.kb1)
      publish_slots(sm.slot[(u.kb0 + 1) % kRing], &sm.valid[(u.kb0 + 1) % kRing], raw1,
                    a.num_slots, tid);
  }
  if (HALF == 0 && g == 0) {
    sm.visrow[rb * 32 + n][0] = vis0;
    sm.visrow[rb * 32 + n][1] = vis1;
  }
  __syncthreads();
  issue_tile<T, DL, DR>(sm.stage[u.kb0 % kStages], sm.slot[u.kb0 % kRing], c_kv, k_pe, wave,
                        lane);
  if constexpr (G::kBF16 && DL == 512 && DR == 64) {
    // The query tile goes through LDS in two passes of 128 rows x 288 dims (the
    // share of one wave of each pair), parked in the two stages the first key
    // tile does not use: every load instruction then reads 1 KiB of
    // consecutive bytes instead of 32-byte pieces of 32 rows.
    constexpr int kQC = 36;                                     // 16-byte chunks per row and pass
    constexpr int kQPerWave = kRowsPerWG * kQC / kWave / kWaves;  // instructions per wave
    constexpr int kQStageChunks = kRowsPerWG / 2 * kQC;          // 64 rows per stage
    static_assert(kQStageChunks * 16 <= G::kStageBytes && kQStageChunks % kWave == 0 &&
                      kQPerWave * kWave * kWaves == kRowsPerWG * kQC && kStep1 - kStep0 == kQC / 2,
                  "query staging");
    unsigned char* qst[2] = {sm.stage[(u.kb0 + 1) % kStages], sm.stage[(u.kb0 + 2) % kStages]};
    const long long row0 = (long long)u.b * QH + (long long)u.rt * kRowsPerWG;
    const long long rlast = (long long)u.b * QH + QH - 1;  // rows past it are clamped, unused
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int i = 0; i < kQPerWave; ++i) {
        const int c0 = (wave * kQPerWave + i) * kWave;  // first chunk of this instruction
        const int c = c0 + lane;
        const int r = c / kQC, j = c - r * kQC;
        long long gr = row0 + r;
        gr = gr < rlast ? gr : rlast;
        // Chunk j of pass p holds dims 288 p + 8 j .. +8 (latent, then rope).
        const T* src = pass == 0 ? q_lat + gr * DL + 8 * j
                       : j < 28  ? q_lat + gr * DL + 288 + 8 * j
                                 : q_pe + gr * DR + 8 * (j - 28);
        const int h = c0 >= kQStageChunks ? 1 : 0;
        dma16(static_cast<const void*>(src), lds_addr(qst[h] + 16 * (c0 - h * kQStageChunks)));
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (HALF == pass) {
        const int row = rb * 32 + n;  // (LDS address space kept explicit: no flat loads)
        const uint32_t qrow = lds_addr(qst[row >> 6]) + (row & 63) * (kQC * 16);
#pragma unroll
        for (int kk = 0; kk < kStep1 - kStep0; ++kk) {
          q[kk] = bf16x8_t{};
          if (row_live) q[kk] = *(const DDT_LDS bf16x8_t*)(uintptr_t)(qrow + 16 * (2 * kk + g));
        }
      }
      __syncthreads();  // the stages are reused by the next pass and the loop
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < kStep1 - kStep0; ++kk) {
      const int d = (kStep0 + kk) * G::kKStep + g * (G::kBF16 ? 8 : 1);
      if constexpr (G::kBF16) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row_live)
          v = d < DL ? *reinterpret_cast<const uint4*>(q_lat + grow * DL + d)
                     : *reinterpret_cast<const uint4*>(q_pe + grow * DR + (d - DL));
        q[kk] = __builtin_bit_cast(bf16x8_t, v);
      } else {
        float v = 0.0f;
        if (row_live) v = d < DL ? q_lat[grow * DL + d] : q_pe[grow * DR + (d - DL)];
        q[kk] = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // State carried between the phases of one tile: the partial scores (QK ->
  // softmax) and the value-product operands (softmax -> PV).
  f32x16_t s = f32x16_t{};
  float p[8];                               // fp32 probabilities of own keys (fp32 inputs)
  bf16x8_t p0 = bf16x8_t{}, p1 = bf16x8_t{};  // keys 0..15 / 16..31 (bf16 inputs)
  bf16x8_t r0 = bf16x8_t{}, r1 = bf16x8_t{};  // their rounding residuals
  bool heavy0 = false, heavy1 = false;
  // The partner's share of the row sum as of its previous tile (a lower bound
  // of its current share), for the residual test.
  float l_mate = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = 0.0f;

  // Partial S^T = K Q^T of tile kb over this wave's share of the contraction.
  auto do_qk = [&](int kb, int lane_it) __attribute__((always_inline)) {
    const int n = lane_it & 31;
    const int g = lane_it >> 5;
    const unsigned char* stg = sm.stage[kb % kStages];
    const T* kt = reinterpret_cast<const T*>(stg);
    const T* kpe = reinterpret_cast<const T*>(stg + G::kLatBytes);
    s = f32x16_t{};
    const T* krow = kt + n * G::kLatPitch + g * (G::kBF16 ? 8 : 1);
    const T* prow = kpe + n * DR;
    const int xswz = g ^ (n & 7);  // rope: physical chunk = logical chunk ^ (n & 7)
    // Permuted latent rows: logical chunk 2*step + g of key n is at byte
    // n*1024 + 16*((2*step + g) ^ swz(n)) = (base ^ 32*(step % 8)) + 256*(step / 8).
    const uint32_t qk_base = lds_addr(kt) + n * G::kLatPitchB + 16 * (g ^ swz(n));
#pragma unroll
    for (int kk = 0; kk < kStep1 - kStep0; ++kk) {
      constexpr int kLatSteps = DL / G::kKStep;
      const int step = kStep0 + kk;
      if constexpr (G::kBF16) {
        bf16x8_t kop;
        if (step < kLatSteps) {
          if constexpr (G::kSwz)
            kop = *(const DDT_LDS bf16x8_t*)(uintptr_t)((qk_base ^ ((step & 7) << 5)) +
                                                        256 * (step >> 3));
          else
            kop = *reinterpret_cast<const bf16x8_t*>(krow + step * 16);
        } else if constexpr (G::kPeChunks == 8) {
          kop = *reinterpret_cast<const bf16x8_t*>(prow + ((2 * (step - kLatSteps)) ^ xswz) * 8);
        } else {
          kop = *reinterpret_cast<const bf16x8_t*>(prow + (step - kLatSteps) * 16 + g * 8);
        }
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, q[kk], s, 0, 0, 0);
      } else {
        const T* src = step < kLatSteps ? krow + step * 2 : prow + (step - kLatSteps) * 2 + g;
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(*src, q[kk], s, 0, 0, 0);
      }
    }
  };

  // Softmax of tile kb over this wave's 16 keys; leaves the value-product
  // operands of all 32 keys in p0/p1 (r0/r1, heavy0/heavy1) or p + xp.
  auto do_softmax = [&](int kb, int lane_it) __attribute__((always_inline)) {
    const int n = lane_it & 31;
    const int g = lane_it >> 5;
    // Lane owns row n and keys 8*(i/4) + 4*g + (i%4) of register i; registers
    // kOwn..kOwn+7 are this wave's keys.  Hand over the partner's, take ours.
    sm.xs[wave][0][lane_it] = make_float4(s[kMate], s[kMate + 1], s[kMate + 2], s[kMate + 3]);
    sm.xs[wave][1][lane_it] = make_float4(s[kMate + 4], s[kMate + 5], s[kMate + 6], s[kMate + 7]);
    pair_post(&sm.xflag[wave], ++seq);
    pair_wait(&sm.xflag[mate], seq, a.spin_limit, stalled);
    float sv[8];
    {
      const float4 h0 = sm.xs[mate][0][lane_it];
      const float4 h1 = sm.xs[mate][1][lane_it];
      sv[0] = s[kOwn] + h0.x;
      sv[1] = s[kOwn + 1] + h0.y;
      sv[2] = s[kOwn + 2] + h0.z;
      sv[3] = s[kOwn + 3] + h0.w;
      sv[4] = s[kOwn + 4] + h1.x;
      sv[5] = s[kOwn + 5] + h1.y;
      sv[6] = s[kOwn + 6] + h1.z;
      sv[7] = s[kOwn + 7] + h1.w;
    }
    // Invisible keys get -inf; the scale (> 0) is applied inside the exponent.
    // Register j of sv is key 16*HALF + 8*(j/4) + 4*g + (j%4).
    const int key0 = kb * kTileKeys;
    const uint32_t valid = (uint32_t)uni((int)sm.valid[kb % kRing]);
    const bool tree_tile = key0 + kTileKeys > u.ri.L;
    if (tree_tile || valid != 0xFFFFFFFFu) {
      uint32_t okm = valid;
      if (tree_tile) {
        const uint64_t* vr = sm.visrow[rb * 32 + n];
        okm &= tree_window(vr[0], vr[1], key0 - u.ri.L);
      }
      okm >>= 16 * HALF + 4 * g;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        sv[j] = ((okm >> (8 * (j >> 2) + (j & 3))) & 1u) ? sv[j] : -INFINITY;
    }
    float mo = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    mo = xor32_max(mo);  // row max over this wave's 16 keys (unscaled)

    // Probabilities of this wave's keys against reference `mref`, posted
    // (with their bf16 residuals when some key of a row is heavy) for the
    // partner.
    float psum = 0.0f;
    bf16x8_t pk = bf16x8_t{}, rk = bf16x8_t{};
    bool heavy = false;
    auto post_p = [&](float mref) __attribute__((always_inline)) {
      psum = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[j], a.sl2, -mref));
        psum += p[j];
      }
      if constexpr (G::kBF16) {
        pk = pack_p<false>(p);
        sm.xp[wave][0][lane_it] = __builtin_bit_cast(float4, pk);
        // Residual pass when some row's largest probability here is a sizeable
        // share of the row's running sum (this wave's keys so far plus the
        // partner's up to its previous tile: a lower bound of the full sum, so
        // the test errs towards the residual).
        const float pmax = __builtin_amdgcn_exp2f(__builtin_fmaf(mo, a.sl2, -mref));
        const float lrow = xor32_sum(l_run + psum) + l_mate;
        heavy = __ballot(pmax > kHeavyShare * lrow) != 0;
        if (heavy) {
          rk = pack_p<true>(p);
          sm.xr[wave][lane_it] = __builtin_bit_cast(uint4, rk);
        }
        sm.xheavy[wave] = heavy ? 1u : 0u;
      } else {
        sm.xp[wave][0][lane_it] = make_float4(p[0], p[1], p[2], p[3]);
        sm.xp[wave][1][lane_it] = make_float4(p[4], p[5], p[6], p[7]);
      }
    };
    post_p(m_run == -INFINITY ? 0.0f : m_run);
    sm.xm[wave][lane_it] = mo;
    if constexpr (G::kBF16) sm.xl[wave][lane_it] = xor32_sum(l_run);
    pair_post(&sm.xflag[wave], ++seq);
    pair_wait(&sm.xflag[mate], seq, a.spin_limit, stalled);
    if constexpr (G::kBF16) l_mate = sm.xl[mate][lane_it];
    // Lazy rescaling: the reference moves on a row's first visible key or
    // when the pair's tile max exceeds it by more than kRescaleLog2, so
    // probabilities stay below 2^kRescaleLog2.  Both waves see the same
    // maxima, so they agree on whether to move.
    const float mt = fmaxf(mo, sm.xm[mate][lane_it]) * a.sl2;
    float m_new = m_run;
    if (m_run == -INFINITY || mt > m_run + kRescaleLog2) m_new = mt;
    if (__ballot(m_new != m_run) != 0) {
      const float alpha =
          (m_run == -INFINITY || m_new == m_run) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      l_mate *= alpha;
      m_run = m_new;
#pragma unroll
      for (int cb = 0; cb < G::kNCBh; ++cb) o[cb] *= alpha;
      post_p(m_run == -INFINITY ? 0.0f : m_run);
      pair_post(&sm.xflag[wave], ++seq);
      pair_wait(&sm.xflag[mate], seq, a.spin_limit, stalled);
    }
    l_run += psum;
    if constexpr (G::kBF16) {
      const bf16x8_t pm = __builtin_bit_cast(bf16x8_t, sm.xp[mate][0][lane_it]);
      const bool heavy_m = uni((int)sm.xheavy[mate]) != 0;
      p0 = HALF == 0 ? pk : pm;
      p1 = HALF == 0 ? pm : pk;
      heavy0 = HALF == 0 ? heavy : heavy_m;
      heavy1 = HALF == 0 ? heavy_m : heavy;
      if (heavy_m) {
        const bf16x8_t rm = __builtin_bit_cast(bf16x8_t, sm.xr[mate][lane_it]);
        r0 = HALF == 0 ? rk : rm;
        r1 = HALF == 0 ? rm : rk;
      } else {
        r0 = rk;
        r1 = rk;
      }
    }
  };

  // O^T += V^T P^T of tile kb over this wave's output columns, keys 0..15
  // (operand of HALF 0) and 16..31 (operand of HALF 1).
  auto do_pv = [&](int kb, int lane_it) __attribute__((always_inline)) {
    const int n = lane_it & 31;
    const int g = lane_it >> 5;
    const T* kt = reinterpret_cast<const T*>(sm.stage[kb % kStages]);
    if constexpr (G::kBF16) {
      const uint16_t* vbase = reinterpret_cast<const uint16_t*>(kt);
      const int colh = 16 * ((lane_it >> 4) & 1);
      // V^T operands: keys k..k+3 (first read) and k+8..k+11 (second) with
      // k = 4g (A0) or 16 + 4g (A1), columns 32*cb + colh + 0..15.
      const VtAddr va(lds_addr(kt), lane_it);
      auto vt = [&](int cb, int k1) -> bf16x8_t {
        if constexpr (G::kSwz) return va.read(kCb0 + cb, k1);
        else return read_vt(vbase, G::kLatPitch, 16 * k1 + 4 * g, (kCb0 + cb) * 32 + colh, lane_it);
      };
#pragma unroll
      for (int cb = 0; cb < G::kNCBh; ++cb) {
        const bf16x8_t a0 = vt(cb, 0);
        const bf16x8_t a1 = vt(cb, 1);
        o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, p0, o[cb], 0, 0, 0);
        o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, p1, o[cb], 0, 0, 0);
      }
      if (heavy0) {
#pragma unroll
        for (int cb = 0; cb < G::kNCBh; ++cb)
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt(cb, 0), r0, o[cb], 0, 0, 0);
      }
      if (heavy1) {
#pragma unroll
        for (int cb = 0; cb < G::kNCBh; ++cb)
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt(cb, 1), r1, o[cb], 0, 0, 0);
      }
    } else {
      float pa[16];
      {
        const float4 m0 = sm.xp[mate][0][lane_it];
        const float4 m1 = sm.xp[mate][1][lane_it];
        const float mp[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pa[kOwn + j] = p[j];
          pa[kMate + j] = mp[j];
        }
      }
#pragma unroll
      for (int cb = 0; cb < G::kNCBh; ++cb) {
        const int c0 = (kCb0 + cb) * 32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = 8 * (i >> 2) + 4 * g + (i & 3);
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kt[m * G::kLatPitch + c0 + n], pa[i],
                                                        o[cb], 0, 0, 0);
        }
      }
    }
  };

  for (int kb = u.kb0; kb < u.kb1; ++kb) {
    // Lane-derived offsets are recomputed every tile from an opaque copy of the
    // lane id: a handful of VALU ops instead of registers held across the loop.
    int lane_it = lane;
    __asm__ __volatile__("" : "+v"(lane_it));
    int32_t ahead = -1;
    if (tid < kTileKeys && kb + 2 < u.kb1)
      ahead = fetch_slot(slots_b, (kb + 2) * kTileKeys + tid, u.nkeys);
    // Tile kb+1 goes to the stage tile kb-2 used (every wave finished it
    // before the previous iteration's closing barrier).
    // The two waves of a pair issue their loads at different points of the
    // iteration, so the CU's load path is not hit by every wave at once.
    const bool dma_next = kb + 1 < u.kb1;
    if (dma_next && (HALF == 0 || !wave_live || kb == u.kb0))
      issue_tile<T, DL, DR>(sm.stage[(kb + 1) % kStages], sm.slot[(kb + 1) % kRing], c_kv, k_pe,
                            wave, lane_it);
    if (wave_live) {
      if (kb > u.kb0) {
        do_pv(kb - 1, lane_it);
        if (HALF == 1 && dma_next)
          issue_tile<T, DL, DR>(sm.stage[(kb + 1) % kStages], sm.slot[(kb + 1) % kRing], c_kv,
                                k_pe, wave, lane_it);
      }
      do_qk(kb, lane_it);
      do_softmax(kb, lane_it);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile kb+1 have landed in LDS
    if (tid < kTileKeys && kb + 2 < u.kb1)
      publish_slots(sm.slot[(kb + 2) % kRing], &sm.valid[(kb + 2) % kRing], ahead, a.num_slots,
                    tid);
    __syncthreads();
  }
  // Drain: the last tile's value product.
  if (wave_live) {
    int lane_it = lane;
    __asm__ __volatile__("" : "+v"(lane_it));
    do_pv(u.kb1 - 1, lane_it);
  }

  // Row sum: this lane's keys, its twin lane's (l ^ 32) and the partner's.
  const float l_own = xor32_sum(l_run);
  sm.xl[wave][lane] = l_own;
  __syncthreads();
  const float l = l_own + sm.xl[mate][lane];
  // Normalise and write: this lane holds row n, columns
  // (kCb0 + cb)*32 + 8*t + 4*g + {0..3} in o[cb][4t..4t+3].
  const float inv = stalled ? __builtin_nanf("") : (l > 0.0f ? 1.0f / l : 0.0f);
  const float lse_v =
      stalled ? __builtin_nanf("") : (l > 0.0f ? (m_run + log2f(l)) * kLn2 : -INFINITY);
  float* dst = nullptr;
  float* dst_lse = nullptr;
  if (u.complete) {
    if (row_exists) {
      dst = a.out + grow * DL;
      dst_lse = a.lse ? a.lse + grow : nullptr;
    }
  } else if (row_live) {
    const long long rr = u.slot * kRowsPerWG + rb * 32 + n;
    dst = a.ws_o + rr * DL;
    dst_lse = a.ws_lse + rr;
  }
  if constexpr (G::kNCBh % 2 == 0) {
    // Rows go out through LDS (the key stages are free now): each pass parks 64
    // of this wave's columns of its 32 rows, then every store instruction
    // writes four 256-byte row segments instead of 32-byte pieces of 32 rows.
    constexpr int kPCb = 2, kPCols = 32 * kPCb, kPitch = kPCols + 4;  // floats
    static_assert(kWaves * 32 * kPitch * 4 <= kStages * G::kStageBytes, "epilogue staging");
    float* buf = reinterpret_cast<float*>(sm.stage[0]) + wave * (32 * kPitch);
    const uint32_t live_m = (uint32_t)__ballot(row_live);  // bit r: row r of this wave
    const uint32_t exist_m = (uint32_t)__ballot(row_exists);
    const uint32_t write_m = u.complete ? exist_m : live_m;
    float* base = u.complete
                      ? a.out + ((long long)u.b * QH + (long long)u.rt * kRowsPerWG + rb * 32) * DL
                      : a.ws_o + ((long long)u.slot * kRowsPerWG + rb * 32) * DL;
    const int c4 = lane & 15;
#pragma unroll
    for (int pass = 0; pass < G::kNCBh / kPCb; ++pass) {
#pragma unroll
      for (int c = 0; c < kPCb; ++c) {
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          const int cb = pass * kPCb + c;
          float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
          if (row_live)
            v = make_float4(o[cb][4 * t4] * inv, o[cb][4 * t4 + 1] * inv,
                            o[cb][4 * t4 + 2] * inv, o[cb][4 * t4 + 3] * inv);
          *reinterpret_cast<float4*>(buf + n * kPitch + c * 32 + 8 * t4 + 4 * g) = v;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's parked rows are in LDS
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4);
        const float4 v = *reinterpret_cast<const float4*>(buf + r * kPitch + 4 * c4);
        float* d = base + (long long)r * DL + (kCb0 + pass * kPCb) * 32 + 4 * c4;
        if ((write_m >> r) & 1u) store_through(d, v);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next pass overwrites
    }
    if (dst_lse && g == 0 && HALF == 0) *dst_lse = row_live ? lse_v : -INFINITY;
  } else if (dst) {
#pragma unroll
    for (int cb = 0; cb < G::kNCBh; ++cb) {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row_live)
          v = make_float4(o[cb][4 * t4] * inv, o[cb][4 * t4 + 1] * inv,
                          o[cb][4 * t4 + 2] * inv, o[cb][4 * t4 + 3] * inv);
        *reinterpret_cast<float4*>(dst + (kCb0 + cb) * 32 + 8 * t4 + 4 * g) = v;
      }
    }
    if (dst_lse && g == 0 && HALF == 0) *dst_lse = row_live ? lse_v : -INFINITY;
  }
}

// The units of the share of the work of workgroup `bl` (0 <= bl < G, or < 2G
// for the aligned split), handed to `run` one by one.  Called by all kThr
// threads of the workgroup; SM provides pref, wsum and req.  The workgroup
// with `write_pref` stores the work prefix and split mode for the merge.
template <int kThr, bool kSplit2, class SM, class Run>
__device__ __forceinline__ void for_each_unit(SM& sm, const int32_t* __restrict__ prefix_len,
                                              const int32_t* __restrict__ n_nodes, int B, int Q,
                                              int H, int max_kv, int RT,
                                              long long* __restrict__ ws_pref, int G,
                                              long long bl, bool write_pref, Run&& run) {
  const long long Gn = G;
  // Launched with 2G workgroups for the aligned split (see workgroup_range);
  // the kernel decides from the clamped request sizes whether it applies.
  const SplitMode sp = work_prefix<kThr>(sm.pref, sm.wsum, sm.req, prefix_len, n_nodes, B, Q, H,
                                         max_kv, RT, Gn, kSplit2);
  const long long Wtot = uni(sm.pref[B]);
  const long long mode = uni(sp.mode);
  const int c = uni(sp.c);
  const bool second = kSplit2 && bl >= Gn;
  if (write_pref) {  // for the merge kernels: stream prefix, split mode, start cost
    for (int i = threadIdx.x; i <= B; i += kThr) ws_pref[i] = sm.pref[i];
    if (threadIdx.x == 0) {
      ws_pref[B + 1] = mode;
      ws_pref[B + 2] = c;
    }
  }
  const long long gid = logical_gid(bl - (second ? Gn : 0), Gn);
  long long start, end;
  const ReqInfo ri0 = req_info_ln(sm.req[0].x, sm.req[0].y, H, RT);
  workgroup_range(mode, second, gid, Wtot, ri0.nkb + c, Gn, start, end);
  start = uni(start);
  end = uni(end);
  if (start >= end) return;

  // Request holding `start`: the last b with pref[b] <= start (it has work).
  int b = 0;
  {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sm.pref[mid] <= start) lo = mid; else hi = mid - 1;
    }
    b = uni(lo);
  }

  // Units of [start, end): the head (holding `start`) may begin mid-row-tile,
  // every later unit begins at key tile 0.  Later units run first and the head
  // last, so that at any moment the workgroups of one XCD (consecutive ranges,
  // mostly the same request) stream nearly the same key tiles and share them
  // in L2 instead of trailing each other by a range's offset.
  // The unit at stream position pos of request b (pref[b] <= pos).
  auto unit_of = [&](long long pos, int b, long long& adv) __attribute__((always_inline)) {
    Unit u;
    u.b = b;
    const int2 ln = sm.req[b];
    u.ri = req_info_ln(uni(ln.x), uni(ln.y), H, RT);
    const UnitPos up = unit_at(pos, end, uni(sm.pref[b]), u.ri, c);
    u.rt = up.rt;
    u.kb0 = up.kb0;
    u.kb1 = up.kb1;
    u.complete = up.complete;
    u.slot = partial_slot(gid, pos == start);
    u.nkeys = u.ri.L + u.ri.nb;
    adv = up.adv;
    return u;
  };
  // The head is computed first (for its length); when later units follow it
  // is computed again after them rather than kept across their runs.
  long long adv;
  Unit u = unit_of(start, b, adv);
  long long pos = start + adv;
  const int b_head = b;
  bool later = pos < end;
  bool head_left = true;
  for (;;) {
    if (later) {
      if (pos < end) {
        while (uni(sm.pref[b + 1]) <= pos) ++b;
        b = uni(b);
        u = unit_of(pos, b, adv);
        pos += adv;
      } else {
        u = unit_of(start, b_head, adv);
        later = false;
        head_left = false;
      }
    } else if (head_left) {
      head_left = false;  // u is the head
    } else {
      break;
    }
    if (u.kb1 <= u.kb0) continue;  // the range ends inside this tile's start cost
    run(u, gid);
  }
}

template <typename T, int DL, int DR, bool kSplit2>
__global__ __launch_bounds__(kThreads) void verify_attn_kernel(
    const T* __restrict__ q_lat, const T* __restrict__ q_pe, const T* __restrict__ c_kv,
    const T* __restrict__ k_pe, int64_t num_slots, const int32_t* __restrict__ req_to_slot,
    int max_kv, const int32_t* __restrict__ prefix_len, const int32_t* __restrict__ n_nodes,
    const uint64_t* __restrict__ vis, int B, int Q, int H, int RT, float sm_scale,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, long long* __restrict__ ws_pref, int G, int spin_limit) {
  __shared__ Smem<T, DL, DR> sm;
  const Args args{q_lat, q_pe, c_kv, k_pe, num_slots, req_to_slot, max_kv, vis, Q, H,
                  sm_scale * kLog2e, out, lse, ws_o, ws_lse, spin_limit};
  const int half = uni((int)((threadIdx.x >> 6) & 1));  // share of the pair: wave % 2
  if ((threadIdx.x & 63) == 0) sm.xflag[threadIdx.x >> 6] = 0;
  int seq = 0;  // this wave's pair-sync sequence (see pair_post)
  for_each_unit<kThreads, kSplit2>(sm, prefix_len, n_nodes, B, Q, H, max_kv, RT, ws_pref, G,
                                   blockIdx.x, blockIdx.x == 0, [&](const Unit& u, long long) __attribute__((always_inline)) {
                                     if (half == 0) run_unit<T, DL, DR, 0>(sm, args, u, seq);
                                     else run_unit<T, DL, DR, 1>(sm, args, u, seq);
                                   });
}

// ----------------------------------------------------------------------------
// Wide form (bf16, 512 + 64): one wavefront per 32 rows, four per workgroup,
// one per SIMD.  Each wave holds its rows' whole query (36 operand registers)
// and whole output (16 accumulator blocks of 32 columns, the 256 accumulator
// registers), so both contractions of a tile run inside one wave and the
// softmax needs no exchange: a row's 32 scores sit in two lanes (l, l ^ 32).
// Per tile a wave issues 36 QK^T and 32 PV MFMAs; the softmax of tile t is
// computed while the value product of tile t-1 runs, so the matrix core of
// the SIMD keeps a queue of independent MFMAs while the VALU works.
constexpr int kWavesW = 4;
constexpr int kThreadsW = kWavesW * kWave;

template <int DL, int DR>
struct SmemW {
  using G = Geo<uint16_t, DL, DR>;
  alignas(1024) unsigned char stage[kStages][G::kStageBytes];
  alignas(16) int32_t slot[kRing][kTileKeys];  // pool slot of each key of a tile (0 when invalid)
  uint32_t valid[kRing];            // bit m: key m of the tile is in range with a valid slot
  uint64_t visrow[kRowsPerWG][2];   // visibility bitset of each row's tree node
  alignas(128) unsigned char qpe[kRowsPerWG][DR * 2];  // rope part of the query tile
  long long pref[kMaxBatch + 1];
  int2 req[kMaxBatch];  // per request: clamped prefix length, tree size
  long long wsum[2 * kWavesW];
};

// Direct loads of one key tile by the four waves: wave w fills the latent rows
// of keys 8w..8w+7 (one 1 KiB row per instruction, the slot read as a scalar)
// and the rope rows of the same keys (one instruction of 8 keys x 8 chunks).
// Measured on gfx950: issuing the nine loads together at the top of the tile
// costs less than spreading them between the MFMAs.
template <int DL, int DR>
__device__ __forceinline__ void issue_tile_w(unsigned char* stage, const int32_t* ring_slots,
                                             const uint16_t* __restrict__ c_kv,
                                             const uint16_t* __restrict__ k_pe, int wave,
                                             int lane) {
  using G = Geo<uint16_t, DL, DR>;
  static_assert(G::kLatChunks == kWave && G::kPeChunks == 8 && G::kLatInstr == 8 * kWavesW &&
                    G::kPeInstr == kWavesW,
                "wide tile loads");
  const int4 s0 = *reinterpret_cast<const int4*>(ring_slots + wave * 8);
  const int4 s1 = *reinterpret_cast<const int4*>(ring_slots + wave * 8 + 4);
  const int pe_row = ring_slots[wave * 8 + (lane >> 3)];
  const int rows[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int key = wave * 8 + it;
    const long long row = uni(rows[it]);
    dma16(static_cast<const void*>(c_kv + row * DL + (lane ^ swz(key)) * G::kPerChunk),
          lds_addr(stage + key * G::kLatPitchB));
  }
  // 8 keys x 8 chunks; key & 7 == lane / 8, so the swizzled chunk depends on
  // the lane only.
  const uint16_t* src = k_pe + (long long)pe_row * DR + (((lane & 7) ^ (lane >> 3)) * G::kPerChunk);
  dma16(static_cast<const void*>(src), lds_addr(stage + G::kLatBytes + wave * kWave * 16));
}

// Reference max of the wide form, in log2 units: a row's reference is the max
// of its first tile with a visible key and does not move afterwards, so the
// accumulators are never rescaled inside the tile loop.  A later score more
// than kOverflowLog2 above it (probabilities up to 2^kOverflowLog2 keep every
// sum far from fp32 overflow) makes the unit run again from its first tile
// with each row's reference at the largest score of the whole range.
constexpr float kOverflowLog2 = 64.0f;

// One step of the score chain S^T += K Q^T with the accumulator in VGPRs, for
// builds whose MFMAs default to AGPR accumulators (all 256 of them hold the
// output).  The hazards the compiler cannot see through the asm are covered
// here: two wait states before each MFMA (a VALU write of an operand just
// before it), back-to-back steps accumulate into the same registers (no wait
// needed), and after the last step the MFMA's result latency is waited out
// before anything may read the scores.
template <bool kFirst, bool kLast>
__device__ __forceinline__ void mfma_qk(f32x16_t& s, bf16x8_t a, bf16x8_t b) {
  if constexpr (kFirst)
    __asm__ __volatile__("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                         : "=&v"(s) : "v"(a), "v"(b));
  else if constexpr (kLast)
    __asm__ __volatile__("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
                         "s_nop 7\n\ts_nop 7\n\ts_nop 5"
                         : "+v"(s) : "v"(a), "v"(b));
  else
    __asm__ __volatile__("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                         : "+v"(s) : "v"(a), "v"(b));
}

template <int DL, int DR>
__device__ __forceinline__ void run_unit_w(SmemW<DL, DR>& sm, const Args& a, const Unit& u) {
  using G = Geo<uint16_t, DL, DR>;
  using T = uint16_t;
  constexpr int kNK = G::kNK;               // QK^T MFMAs per tile (576 / 16)
  constexpr int kLatSteps = DL / G::kKStep;  // ... of them over the latent part
  constexpr int kNCB = G::kNCB;             // 32-column output blocks
  static_assert(G::kSwz && DR == 64 && kNK == 36 && kNCB == 16 && kLatSteps == 32,
                "wide form shape");
  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6);
  int lane = tid;
  __asm__ __volatile__("" : "+v"(lane));
  lane &= 63;
  const int n = lane & 31;
  const int g = lane >> 5;
  const int W = (a.Q + 63) >> 6;
  const long long QH = (long long)a.Q * a.H;
  const T* q_lat = static_cast<const T*>(a.q_lat);
  const T* q_pe = static_cast<const T*>(a.q_pe);
  const T* c_kv = static_cast<const T*>(a.c_kv);
  const T* k_pe = static_cast<const T*>(a.k_pe);
  const int32_t* slots_b = a.req_to_slot + (long long)u.b * a.max_kv;

  const int rloc = wave * 32 + n;  // row within the tile
  const long long r_loc = (long long)u.rt * kRowsPerWG + rloc;
  int heads = a.H;
  __asm__ __volatile__("" : "+s"(heads));
  const int node = (int)(r_loc / heads);
  const bool row_exists = r_loc < QH;
  const bool row_live = row_exists && node < u.ri.nb;
  const bool wave_live = __ballot(row_live) != 0;

  // Slot ids of the unit's first two tiles, published to the ring, then the
  // first tile's loads (done again when the unit restarts).
  auto start_tiles = [&]() __attribute__((always_inline)) {
    int32_t raw0 = -1, raw1 = -1;
    if (tid < kTileKeys) {
      raw0 = fetch_slot(slots_b, u.kb0 * kTileKeys + tid, u.nkeys);
      if (u.kb0 + 1 < u.kb1) raw1 = fetch_slot(slots_b, (u.kb0 + 1) * kTileKeys + tid, u.nkeys);
      publish_slots(sm.slot[u.kb0 % kRing], &sm.valid[u.kb0 % kRing], raw0, a.num_slots, tid);
      if (u.kb0 + 1 < u.kb1)
        publish_slots(sm.slot[(u.kb0 + 1) % kRing], &sm.valid[(u.kb0 + 1) % kRing], raw1,
                      a.num_slots, tid);
    }
  };

  uint64_t vis0 = 0, vis1 = 0;
  if (g == 0 && row_live) {
    const uint64_t* vr = a.vis + ((long long)u.b * a.Q + node) * W;
    vis0 = vr[0];
    if (W > 1) vis1 = vr[1];
  }
  start_tiles();
  if (g == 0) {
    sm.visrow[rloc][0] = vis0;
    sm.visrow[rloc][1] = vis1;
  }
  __syncthreads();
  issue_tile_w<DL, DR>(sm.stage[u.kb0 % kStages], sm.slot[u.kb0 % kRing], c_kv, k_pe, wave, lane);

  // The latent query tile goes through LDS in two passes (dims 0..287, then
  // 288..511) of 128 rows, parked in the two stages the first key tile does
  // not use, and is read into registers; each load instruction reads 1 KiB of
  // consecutive bytes.  The rope part stays in LDS (qpe), where the score
  // MFMAs read it like the keys' rope rows.
  bf16x8_t q[kLatSteps];
  {
    unsigned char* qst[2] = {sm.stage[(u.kb0 + 1) % kStages], sm.stage[(u.kb0 + 2) % kStages]};
    const long long row0 = (long long)u.b * QH + (long long)u.rt * kRowsPerWG;
    const long long rlast = (long long)u.b * QH + QH - 1;  // rows past it are clamped, unused
    {
      // Rope rows: 8 rows x 8 chunks per instruction, chunk c of row r stored
      // at chunk c ^ (r & 7); rows 8i..8i+7 by instruction i.
      constexpr int kPerWave = kRowsPerWG / 8 / kWavesW;
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        const int r = (wave * kPerWave + i) * 8 + (lane >> 3);
        long long gr = row0 + r;
        gr = gr < rlast ? gr : rlast;
        const T* src = q_pe + gr * DR + (((lane & 7) ^ (lane >> 3)) * G::kPerChunk);
        dma16(static_cast<const void*>(src), lds_addr(&sm.qpe[(wave * kPerWave + i) * 8][0]));
      }
    }
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int kQC = pass == 0 ? 36 : 28;                      // 16-byte chunks per row
      const int kQPerWave = kRowsPerWG * kQC / kWave / kWavesW;  // instructions per wave
      const int kQStageChunks = kRowsPerWG / 2 * kQC;             // 64 rows per stage
#pragma unroll
      for (int i = 0; i < kQPerWave; ++i) {
        const int c0 = (wave * kQPerWave + i) * kWave;  // first chunk of this instruction
        const int c = c0 + lane;
        const int r = c / kQC, j = c - r * kQC;
        long long gr = row0 + r;
        gr = gr < rlast ? gr : rlast;
        // Chunk j of pass p holds dims 288 p + 8 j .. +8.
        const T* src = q_lat + gr * DL + 288 * pass + 8 * j;
        const int h = c0 >= kQStageChunks ? 1 : 0;
        dma16(static_cast<const void*>(src), lds_addr(qst[h] + 16 * (c0 - h * kQStageChunks)));
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const uint32_t qrow = lds_addr(qst[rloc >> 6]) + (rloc & 63) * (kQC * 16);
#pragma unroll
      for (int kk = 0; kk < kQC / 2; ++kk) {
        q[18 * pass + kk] = bf16x8_t{};
        if (row_live)
          q[18 * pass + kk] = *(const DDT_LDS bf16x8_t*)(uintptr_t)(qrow + 16 * (2 * kk + g));
      }
      __syncthreads();  // the stages are reused by the next pass and the loop
    }
  }

  constexpr int kAhead = 4;    // score operand reads in flight ahead of the MFMAs
  constexpr int kAheadPV = 6;  // value operand reads in flight ahead of the MFMAs

  // m_ref: the row's reference max (log2 units), the same in both lanes of the
  // row; m_seen: the largest scaled score so far; l_run: this lane's share of
  // the row sum (its 16 keys of each tile).
  float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.0f;
  bool overflow = false;

  // The softmax of a tile runs one tile late, in parts placed between the
  // MFMAs of the next tile's QK^T (part A: row maxima, reference,
  // probabilities) and of its own value product (part B: row sum and
  // residual test), so the VALU work issues while the matrix core runs.  sv
  // holds the tile's scores until the next tile's replace them; the fences
  // keep each part where it is placed.
  float sv[16];
  float p[16];
  float mh0 = 0.0f, mh1 = 0.0f, mref = 0.0f, psum = 0.0f;
  bf16x8_t p0 = bf16x8_t{}, p1 = bf16x8_t{};
  bool h0 = false, h1 = false;
  auto part_a = [&](int j) __attribute__((always_inline)) {
    if (j == 0) {
      mh0 = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                  fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mh1 = fmaxf(fmaxf(fmaxf(sv[8], sv[9]), fmaxf(sv[10], sv[11])),
                  fmaxf(fmaxf(sv[12], sv[13]), fmaxf(sv[14], sv[15])));
    } else if (j == 1) {
      // Maxima of the row over keys 0..15 and 16..31 (unscaled).
      mh0 = xor32_max(mh0);
      mh1 = xor32_max(mh1);
      const float mt = fmaxf(mh0, mh1) * a.sl2;  // row max over the tile, log2 units
      m_seen = fmaxf(m_seen, mt);
      if (m_ref == -INFINITY) m_ref = mt;  // first visible key of the row (o is still 0)
      overflow = overflow || mt > m_ref + kOverflowLog2;
      mref = m_ref == -INFINITY ? 0.0f : m_ref;
    } else if (j < 10) {
      const int k = 2 * (j - 2);
      p[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[k], a.sl2, -mref));
      p[k + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[k + 1], a.sl2, -mref));
    } else if (j == 10) {
      p0 = pack_p<false>(p);
    } else if (j == 11) {
      p1 = pack_p<false>(p + 8);
    } else if (j == 12) {
      psum = (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]))) +
             (((p[8] + p[9]) + (p[10] + p[11])) + ((p[12] + p[13]) + (p[14] + p[15])));
    }
  };
  constexpr int kPartsA = 13;
  auto part_b = [&](int j) __attribute__((always_inline)) {
    if (j == 0) {
      // Residual pass when some key's probability is a sizeable share of its
      // row's running sum (a lower bound of the final sum, so the test errs
      // towards the residual).
      l_run += psum;
      const float lrow = xor32_sum(l_run);
      const float pm0 = __builtin_amdgcn_exp2f(__builtin_fmaf(mh0, a.sl2, -mref));
      const float pm1 = __builtin_amdgcn_exp2f(__builtin_fmaf(mh1, a.sl2, -mref));
      h0 = __ballot(pm0 > kHeavyShare * lrow) != 0;
      h1 = __ballot(pm1 > kHeavyShare * lrow) != 0;
    }
  };
  constexpr int kPartsB = 1;

  // Invisible keys of tile kb get -inf in sv (prefix keys are always visible;
  // a tree key when its bit is set in the row's node bitset; keys past the
  // request or with an invalid slot never).  The scale (> 0) is applied
  // inside the exponent.  Register i of sv is key 8*(i/4) + 4*g + (i%4).
  auto mask = [&](int kb, int lane_it) __attribute__((always_inline)) {
    const int key0 = kb * kTileKeys;
    const uint32_t valid = (uint32_t)uni((int)sm.valid[kb % kRing]);
    const bool tree_tile = key0 + kTileKeys > u.ri.L;
    if (tree_tile || valid != 0xFFFFFFFFu) {
      const int n = lane_it & 31;
      const int g = lane_it >> 5;
      uint32_t okm = valid;
      if (tree_tile) {
        const uint64_t* vr = sm.visrow[wave * 32 + n];
        okm &= tree_window(vr[0], vr[1], key0 - u.ri.L);
      }
      okm >>= 4 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        sv[i] = ((okm >> (8 * (i >> 2) + (i & 3))) & 1u) ? sv[i] : -INFINITY;
    }
  };

  // S^T = K Q^T of tile kb over all 576 dims, into sv; part A of the previous
  // tile's softmax runs between its MFMAs when `soft` (whose scores sv holds
  // until the chain's result replaces them).  Operand reads run kAhead MFMAs
  // ahead; the fences keep that order (the register budget would otherwise
  // make the scheduler wait for every read).
  auto do_qk = [&](int kb, int lane_it, auto kSoft) __attribute__((always_inline)) {
    constexpr bool soft = decltype(kSoft)::value;
    const int n = lane_it & 31;
    const int g = lane_it >> 5;
    const uint32_t kt = lds_addr(sm.stage[kb % kStages]);
    // Permuted latent rows: logical chunk 2*step + g of key n is at byte
    // n*1024 + 16*((2*step + g) ^ swz(n)) = (base ^ 32*(step % 8)) + 256*(step / 8).
    const uint32_t qk_base = kt + n * G::kLatPitchB + 16 * (g ^ swz(n));
    // Rope rows (keys and queries alike): logical chunk c of row n at
    // physical chunk c ^ (n & 7); query row wave*32 + n has the same n & 7.
    // Rope step k: logical chunk 2k + g at byte 16 * ((2k) ^ xswz) = base ^ 32k.
    const int xswz = g ^ (n & 7);
    const uint32_t pe_base = kt + G::kLatBytes + n * (DR * 2) + 16 * xswz;
    const uint32_t qpe_base = lds_addr(&sm.qpe[wave * 32 + n][0]) + 16 * xswz;
    auto kread = [&](int step) __attribute__((always_inline)) -> bf16x8_t {
      if (step < kLatSteps)
        return *(const DDT_LDS bf16x8_t*)(uintptr_t)((qk_base ^ ((step & 7) << 5)) +
                                                     256 * (step >> 3));
      return *(const DDT_LDS bf16x8_t*)(uintptr_t)(pe_base ^ (32 * (step - kLatSteps)));
    };
    auto qread = [&](int step) __attribute__((always_inline)) -> bf16x8_t {
      if (step < kLatSteps) return q[step];
      return *(const DDT_LDS bf16x8_t*)(uintptr_t)(qpe_base ^ (32 * (step - kLatSteps)));
    };
    bf16x8_t kop[kNK], qop[kNK];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      kop[i] = kread(i);
      qop[i] = qread(i);
    }
    f32x16_t s;
#pragma unroll
    for (int step = 0; step < kNK; ++step) {
      if (step + kAhead < kNK) {
        kop[step + kAhead] = kread(step + kAhead);
        qop[step + kAhead] = qread(step + kAhead);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (step == 0) mfma_qk<true, false>(s, kop[step], qop[step]);
      else if (step == kNK - 1) mfma_qk<false, true>(s, kop[step], qop[step]);
      else mfma_qk<false, false>(s, kop[step], qop[step]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (soft) {
        if (step >= 2 && step % 2 == 0 && (step - 2) / 2 < kPartsA) part_a((step - 2) / 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = s[i];
  };

  f32x16_t o[kNCB];
  // O^T += V^T P^T of tile kb over all 512 columns, part B of its softmax
  // between the MFMAs.  MFMA i: column block i % 16, keys 16 * (i / 16) .. +15
  // (probabilities p0, then p1), so consecutive MFMAs accumulate into
  // different blocks.
  auto do_pv = [&](int kb, int lane_it) __attribute__((always_inline)) {
    const VtAddr va(lds_addr(sm.stage[kb % kStages]), lane_it);
    bf16x8_t vop[2 * kNCB];
#pragma unroll
    for (int i = 0; i < kAheadPV; ++i) vop[i] = va.read(i % kNCB, i / kNCB);
#pragma unroll
    for (int i = 0; i < 2 * kNCB; ++i) {
      if (i + kAheadPV < 2 * kNCB)
        vop[i + kAheadPV] = va.read((i + kAheadPV) % kNCB, (i + kAheadPV) / kNCB);
      __builtin_amdgcn_sched_barrier(0);
      o[i % kNCB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[i], (i / kNCB) ? p1 : p0,
                                                           o[i % kNCB], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (i % 4 == 3 && i / 4 < kPartsB) part_b(i / 4);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Residual pass: (p - bf16(p)) of the key halves that hold a heavy key,
    // through the same V^T operands, read kAheadPV MFMAs ahead.
    auto residual = [&](int k1, const bf16x8_t r) __attribute__((always_inline)) {
      bf16x8_t vr[kNCB];
#pragma unroll
      for (int cb = 0; cb < kAheadPV; ++cb) vr[cb] = va.read(cb, k1);
#pragma unroll
      for (int cb = 0; cb < kNCB; ++cb) {
        if (cb + kAheadPV < kNCB) vr[cb + kAheadPV] = va.read(cb + kAheadPV, k1);
        __builtin_amdgcn_sched_barrier(0);
        o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[cb], r, o[cb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (h0) residual(0, pack_p<true>(p));
    if (h1) residual(1, pack_p<true>(p + 8));
  };

  // Step kb: QK^T of tile kb (with part A of tile kb-1's softmax), then the
  // value product of tile kb-1 (with part B); the unit's first step has no
  // previous tile.
  auto step = [&](int kb, auto kFirst) __attribute__((always_inline)) {
    constexpr bool first = decltype(kFirst)::value;
    // Lane-derived offsets are recomputed every tile from an opaque copy of the
    // lane id: a handful of VALU ops instead of registers held across the loop.
    int lane_it = lane;
    __asm__ __volatile__("" : "+v"(lane_it));
    int32_t ahead = -1;
    if (tid < kTileKeys && kb + 2 < u.kb1)
      ahead = fetch_slot(slots_b, (kb + 2) * kTileKeys + tid, u.nkeys);
    // Tile kb+1 goes to the stage tile kb-2 used (every wave finished it
    // before the previous iteration's closing barrier).
    if (kb + 1 < u.kb1)
      issue_tile_w<DL, DR>(sm.stage[(kb + 1) % kStages], sm.slot[(kb + 1) % kRing], c_kv, k_pe,
                           wave, lane_it);
    if (wave_live) {
      if constexpr (first) {
        do_qk(kb, lane_it, std::false_type{});
      } else {
        mask(kb - 1, lane_it);
        do_qk(kb, lane_it, std::true_type{});  // tile kb's scores replace sv at its end
        do_pv(kb - 1, lane_it);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile kb+1 have landed in LDS
    if (tid < kTileKeys && kb + 2 < u.kb1)
      publish_slots(sm.slot[(kb + 2) % kRing], &sm.valid[(kb + 2) % kRing], ahead, a.num_slots,
                    tid);
    __syncthreads();
  };

  for (int attempt = 0;; ++attempt) {
#pragma unroll
    for (int cb = 0; cb < kNCB; ++cb) o[cb] = f32x16_t{};
    l_run = 0.0f;
    if (attempt > 0) {
      // The rerun: references at each row's largest score, which no tile of
      // the range exceeds.
      m_ref = m_seen;
      start_tiles();
      __syncthreads();
      issue_tile_w<DL, DR>(sm.stage[u.kb0 % kStages], sm.slot[u.kb0 % kRing], c_kv, k_pe, wave,
                           lane);
      __builtin_amdgcn_s_waitcnt(0);  // the first tile is in LDS before its scores are read
      __syncthreads();
    }
    step(u.kb0, std::true_type{});
    for (int kb = u.kb0 + 1; kb < u.kb1; ++kb) step(kb, std::false_type{});
    // Drain: the last tile's softmax and value product.
    if (wave_live) {
      int lane_it = lane;
      __asm__ __volatile__("" : "+v"(lane_it));
      mask(u.kb1 - 1, lane_it);
#pragma unroll
      for (int j = 0; j < kPartsA; ++j) part_a(j);
      do_pv(u.kb1 - 1, lane_it);
    }
    // Every wave's last value product has read the key stages before the
    // epilogue (or a rerun) writes them.
    if (!__syncthreads_or(attempt == 0 && overflow)) break;
    overflow = false;
  }

  // Row sum over the two lanes of the row.
  const float l = xor32_sum(l_run);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const float lse_v = l > 0.0f ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
  float* dst_lse = nullptr;
  if (u.complete) {
    if (row_exists && a.lse) dst_lse = a.lse + (long long)u.b * QH + r_loc;
  } else if (row_live) {
    dst_lse = a.ws_lse + u.slot * kRowsPerWG + rloc;
  }
  // Rows go out through LDS (the key stages are free now): each pass parks 64
  // columns of this wave's 32 rows, then every store instruction writes four
  // 256-byte row segments.
  constexpr int kPCb = 2, kPCols = 32 * kPCb, kPitch = kPCols + 4;  // floats
  static_assert(kWavesW * 32 * kPitch * 4 <= kStages * G::kStageBytes, "epilogue staging");
  float* buf = reinterpret_cast<float*>(sm.stage[0]) + wave * (32 * kPitch);
  const uint32_t live_m = (uint32_t)__ballot(row_live);  // bit r: row r of this wave
  const uint32_t exist_m = (uint32_t)__ballot(row_exists);
  const uint32_t write_m = u.complete ? exist_m : live_m;
  float* base = u.complete
                    ? a.out + ((long long)u.b * QH + (long long)u.rt * kRowsPerWG + wave * 32) * DL
                    : a.ws_o + ((long long)u.slot * kRowsPerWG + wave * 32) * DL;
  const int c4 = lane & 15;
#pragma unroll
  for (int pass = 0; pass < kNCB / kPCb; ++pass) {
#pragma unroll
    for (int c = 0; c < kPCb; ++c) {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int cb = pass * kPCb + c;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row_live)
          v = make_float4(o[cb][4 * t4] * inv, o[cb][4 * t4 + 1] * inv, o[cb][4 * t4 + 2] * inv,
                          o[cb][4 * t4 + 3] * inv);
        *reinterpret_cast<float4*>(buf + n * kPitch + c * 32 + 8 * t4 + 4 * g) = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's parked rows are in LDS
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4);
      const float4 v = *reinterpret_cast<const float4*>(buf + r * kPitch + 4 * c4);
      float* d = base + (long long)r * DL + pass * kPCols + 4 * c4;
      if ((write_m >> r) & 1u) store_through(d, v);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next pass overwrites
  }
  if (dst_lse && g == 0) *dst_lse = row_live ? lse_v : -INFINITY;
}

template <int DL, int DR, bool kSplit2>
__global__ __launch_bounds__(kThreadsW, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void verify_attn_wide_kernel(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ q_pe,
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe, int64_t num_slots,
    const int32_t* __restrict__ req_to_slot, int max_kv, const int32_t* __restrict__ prefix_len,
    const int32_t* __restrict__ n_nodes, const uint64_t* __restrict__ vis, int B, int Q, int H,
    int RT, float sm_scale, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, long long* __restrict__ ws_pref,
    int G) {
  __shared__ SmemW<DL, DR> sm;
  const Args args{q_lat, q_pe, c_kv, k_pe, num_slots, req_to_slot, max_kv, vis, Q, H,
                  sm_scale * kLog2e, out, lse, ws_o, ws_lse, 0};
  for_each_unit<kThreadsW, kSplit2>(sm, prefix_len, n_nodes, B, Q, H, max_kv, RT, ws_pref, G,
                                    blockIdx.x, blockIdx.x == 0, [&](const Unit& u, long long) __attribute__((always_inline)) {
                                      run_unit_w<DL, DR>(sm, args, u);
                                    });
}

// ----------------------------------------------------------------------------
// Narrow form (bf16, 512 + 64, few row tiles): four workgroups share each work
// range, one per 32-row quarter of its row tiles.  Inside a workgroup the four
// waves (one per SIMD) split the contraction of QK^T, nine MFMA steps each, and
// the output columns, 128 each.  The partial scores meet in LDS once per tile;
// every wave sums them in the same order and runs the same softmax, then
// multiplies by its own 128 value columns.  A workgroup holds a quarter of the
// rows of the wide form, so a row tile can be cut into a quarter as many key
// ranges for the same number of busy CUs; at small batches that is what
// bounds the call: partial rows written, flushed at the kernel's end and read
// again by the merge.
constexpr int kStepsN = 9;  // QK^T MFMA steps per wave (36 / 4)
constexpr int kNCBn = 4;    // 32-column output blocks per wave (16 / 4)

template <int DL, int DR>
struct SmemN {
  using G = Geo<uint16_t, DL, DR>;
  alignas(1024) unsigned char stage[kStages][G::kStageBytes];
  float4 sx[2][kWavesW][4][kWave];  // partial scores of each wave, by tile parity
  alignas(16) int32_t slot[kRing][kTileKeys];  // pool slot of each key of a tile (0 when invalid)
  uint32_t valid[kRing];            // bit m: key m of the tile is in range with a valid slot
  uint64_t visrow[32][2];           // visibility bitset of each row's tree node
  long long pref[kMaxBatch + 1];
  int2 req[kMaxBatch];  // per request: clamped prefix length, tree size
  long long wsum[2 * kWavesW];
};

template <int DL, int DR>
__device__ __forceinline__ void run_unit_n(SmemN<DL, DR>& sm, const Args& a, const Unit& u,
                                           int quarter) {
  using G = Geo<uint16_t, DL, DR>;
  using T = uint16_t;
  constexpr int kLatSteps = DL / G::kKStep;  // QK^T steps over the latent part
  static_assert(G::kSwz && DR == 64 && G::kNK == kWavesW * kStepsN &&
                    G::kNCB == kWavesW * kNCBn && kLatSteps == 32,
                "narrow form shape");
  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6);
  int lane = tid;
  __asm__ __volatile__("" : "+v"(lane));
  lane &= 63;
  const int n = lane & 31;
  const int g = lane >> 5;
  const int W = (a.Q + 63) >> 6;
  const long long QH = (long long)a.Q * a.H;
  const T* q_lat = static_cast<const T*>(a.q_lat);
  const T* q_pe = static_cast<const T*>(a.q_pe);
  const T* c_kv = static_cast<const T*>(a.c_kv);
  const T* k_pe = static_cast<const T*>(a.k_pe);
  const int32_t* slots_b = a.req_to_slot + (long long)u.b * a.max_kv;

  // Every wave holds the same 32 rows: row n of the quarter in lanes n, n + 32.
  const int rloc = quarter * 32 + n;  // row within the tile
  const long long r_loc = (long long)u.rt * kRowsPerWG + rloc;
  int heads = a.H;
  __asm__ __volatile__("" : "+s"(heads));
  const int node = (int)(r_loc / heads);
  const bool row_exists = r_loc < QH;
  const bool row_live = row_exists && node < u.ri.nb;
  const bool live = __ballot(row_live) != 0;  // the same in every wave

  float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.0f;
  f32x16_t o[kNCBn];
#pragma unroll
  for (int c = 0; c < kNCBn; ++c) o[c] = f32x16_t{};

  if (live) {
    auto start_tiles = [&]() __attribute__((always_inline)) {
      int32_t raw0 = -1, raw1 = -1;
      if (tid < kTileKeys) {
        raw0 = fetch_slot(slots_b, u.kb0 * kTileKeys + tid, u.nkeys);
        if (u.kb0 + 1 < u.kb1) raw1 = fetch_slot(slots_b, (u.kb0 + 1) * kTileKeys + tid, u.nkeys);
        publish_slots(sm.slot[u.kb0 % kRing], &sm.valid[u.kb0 % kRing], raw0, a.num_slots, tid);
        if (u.kb0 + 1 < u.kb1)
          publish_slots(sm.slot[(u.kb0 + 1) % kRing], &sm.valid[(u.kb0 + 1) % kRing], raw1,
                        a.num_slots, tid);
      }
    };
    uint64_t vis0 = 0, vis1 = 0;
    if (wave == 0 && g == 0 && row_live) {
      const uint64_t* vr = a.vis + ((long long)u.b * a.Q + node) * W;
      vis0 = vr[0];
      if (W > 1) vis1 = vr[1];
    }
    start_tiles();
    if (wave == 0 && g == 0) {
      sm.visrow[n][0] = vis0;
      sm.visrow[n][1] = vis1;
    }
    __syncthreads();
    issue_tile_w<DL, DR>(sm.stage[u.kb0 % kStages], sm.slot[u.kb0 % kRing], c_kv, k_pe, wave,
                         lane);

    // This wave's query operands (steps 9w .. 9w+8: latent chunk 2s + g of
    // the row for s < 32, rope chunk 2(s - 32) + g after), straight from
    // global memory.
    bf16x8_t q[kStepsN];
    {
      long long gr = (long long)u.b * QH + r_loc;
      const long long rlast = (long long)u.b * QH + QH - 1;  // rows past it are unused
      gr = gr < rlast ? gr : rlast;
#pragma unroll
      for (int k = 0; k < kStepsN; ++k) {
        const int st = kStepsN * wave + k;
        const T* src = st < kLatSteps ? q_lat + gr * DL + 16 * st + 8 * g
                                      : q_pe + gr * DR + 16 * (st - kLatSteps) + 8 * g;
        q[k] = row_live ? *reinterpret_cast<const bf16x8_t*>(src) : bf16x8_t{};
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the first tile is in LDS
    __syncthreads();

    bool overflow = false;
    float sv[16];
    float p[16];
    float4 gs[kWavesW][4];  // the four waves' partial scores of the previous tile
    float mh0 = 0.0f, mh1 = 0.0f, mref = 0.0f, psum = 0.0f;
    bf16x8_t p0 = bf16x8_t{}, p1 = bf16x8_t{};
    bool h0 = false, h1 = false;

    // Invisible keys of tile kb get -inf in sv (see the wide form's mask).
    auto mask = [&](int kb, int lane_it) __attribute__((always_inline)) {
      const int key0 = kb * kTileKeys;
      const uint32_t valid = (uint32_t)uni((int)sm.valid[kb % kRing]);
      const bool tree_tile = key0 + kTileKeys > u.ri.L;
      if (tree_tile || valid != 0xFFFFFFFFu) {
        const int nn = lane_it & 31;
        const int gg = lane_it >> 5;
        uint32_t okm = valid;
        if (tree_tile) {
          const uint64_t* vr = sm.visrow[nn];
          okm &= tree_window(vr[0], vr[1], key0 - u.ri.L);
        }
        okm >>= 4 * gg;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sv[i] = ((okm >> (8 * (i >> 2) + (i & 3))) & 1u) ? sv[i] : -INFINITY;
      }
    };

    // The softmax of tile kb-1 in parts, placed between the score MFMAs of
    // tile kb: the four partial scores added in wave order and masked, row
    // maxima and the fixed reference (as in the wide form), probabilities,
    // operands, row sum and the residual test.
    auto part = [&](int j, int kbp, int lane_it) __attribute__((always_inline)) {
      if (j == 0) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          float4 acc = gs[0][i4];
#pragma unroll
          for (int w = 1; w < kWavesW; ++w) {
            acc.x += gs[w][i4].x;
            acc.y += gs[w][i4].y;
            acc.z += gs[w][i4].z;
            acc.w += gs[w][i4].w;
          }
          sv[4 * i4] = acc.x;
          sv[4 * i4 + 1] = acc.y;
          sv[4 * i4 + 2] = acc.z;
          sv[4 * i4 + 3] = acc.w;
        }
        mask(kbp, lane_it);
      } else if (j == 1) {
        mh0 = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                    fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        mh1 = fmaxf(fmaxf(fmaxf(sv[8], sv[9]), fmaxf(sv[10], sv[11])),
                    fmaxf(fmaxf(sv[12], sv[13]), fmaxf(sv[14], sv[15])));
        mh0 = xor32_max(mh0);
        mh1 = xor32_max(mh1);
        const float mt = fmaxf(mh0, mh1) * a.sl2;  // row max over the tile, log2 units
        m_seen = fmaxf(m_seen, mt);
        if (m_ref == -INFINITY) m_ref = mt;
        overflow = overflow || mt > m_ref + kOverflowLog2;
        mref = m_ref == -INFINITY ? 0.0f : m_ref;
      } else if (j < 6) {
        const int k = 4 * (j - 2);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          p[k + t] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[k + t], a.sl2, -mref));
      } else if (j == 6) {
        p0 = pack_p<false>(p);
        p1 = pack_p<false>(p + 8);
      } else if (j == 7) {
        psum = (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]))) +
               (((p[8] + p[9]) + (p[10] + p[11])) + ((p[12] + p[13]) + (p[14] + p[15])));
        l_run += psum;
        const float lrow = xor32_sum(l_run);
        const float pm0 = __builtin_amdgcn_exp2f(__builtin_fmaf(mh0, a.sl2, -mref));
        const float pm1 = __builtin_amdgcn_exp2f(__builtin_fmaf(mh1, a.sl2, -mref));
        h0 = __ballot(pm0 > kHeavyShare * lrow) != 0;
        h1 = __ballot(pm1 > kHeavyShare * lrow) != 0;
      }
    };
    constexpr int kParts = 8;

    // The four waves' partial scores of tile kb (stored before the barrier
    // that ended the step of tile kb), read into gs.
    auto gather = [&](int kb, int lane_it) __attribute__((always_inline)) {
#pragma unroll
      for (int w = 0; w < kWavesW; ++w)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) gs[w][i4] = sm.sx[kb & 1][w][i4][lane_it];
    };

    // This wave's nine steps of S^T = K Q^T for tile kb, stored to LDS; with
    // `soft`, the softmax of tile kb-1 runs between them.
    auto do_qk = [&](int kb, int lane_it, auto kSoft) __attribute__((always_inline)) {
      constexpr bool soft = decltype(kSoft)::value;
      const int nn = lane_it & 31;
      const int gg = lane_it >> 5;
      const uint32_t kt = lds_addr(sm.stage[kb % kStages]);
      const uint32_t qk_base = kt + nn * G::kLatPitchB + 16 * (gg ^ swz(nn));
      const int xswz = gg ^ (nn & 7);
      const uint32_t pe_base = kt + G::kLatBytes + nn * (DR * 2) + 16 * xswz;
      auto kread = [&](int st) __attribute__((always_inline)) -> bf16x8_t {
        if (st < kLatSteps)
          return *(const DDT_LDS bf16x8_t*)(uintptr_t)((qk_base ^ ((st & 7) << 5)) +
                                                       256 * (st >> 3));
        return *(const DDT_LDS bf16x8_t*)(uintptr_t)(pe_base ^ (32 * (st - kLatSteps)));
      };
      bf16x8_t kop[kStepsN];
#pragma unroll
      for (int k = 0; k < kStepsN; ++k) kop[k] = kread(kStepsN * wave + k);
      if constexpr (soft) gather(kb - 1, lane_it);
      f32x16_t s;
#pragma unroll
      for (int k = 0; k < kStepsN; ++k) {
        __builtin_amdgcn_sched_barrier(0);
        if (k == 0) mfma_qk<true, false>(s, kop[k], q[k]);
        else if (k == kStepsN - 1) mfma_qk<false, true>(s, kop[k], q[k]);
        else mfma_qk<false, false>(s, kop[k], q[k]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (soft) {
          if (k < kParts) part(k, kb - 1, lane_it);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      float4* dst = &sm.sx[kb & 1][wave][0][lane_it];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        dst[i4 * kWave] = make_float4(s[4 * i4], s[4 * i4 + 1], s[4 * i4 + 2], s[4 * i4 + 3]);
    };

    // O^T += V^T P^T of tile kb over this wave's 128 columns (blocks 4w..4w+3).
    auto do_pv = [&](int kb, int lane_it) __attribute__((always_inline)) {
      const VtAddr va(lds_addr(sm.stage[kb % kStages]), lane_it);
      bf16x8_t vop[2 * kNCBn];
#pragma unroll
      for (int i = 0; i < 2 * kNCBn; ++i) vop[i] = va.read(kNCBn * wave + i % kNCBn, i / kNCBn);
#pragma unroll
      for (int i = 0; i < 2 * kNCBn; ++i)
        o[i % kNCBn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[i], (i / kNCBn) ? p1 : p0,
                                                               o[i % kNCBn], 0, 0, 0);
      // Residual pass of the key halves with a heavy key: all of a half's
      // operand reads are issued before its MFMAs.
      auto residual = [&](int k1, const bf16x8_t r) __attribute__((always_inline)) {
        bf16x8_t vr[kNCBn];
#pragma unroll
        for (int c = 0; c < kNCBn; ++c) vr[c] = va.read(kNCBn * wave + c, k1);
#pragma unroll
        for (int c = 0; c < kNCBn; ++c)
          o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[c], r, o[c], 0, 0, 0);
      };
      if (h0) residual(0, pack_p<true>(p));
      if (h1) residual(1, pack_p<true>(p + 8));
    };

    // Step kb: tile kb+1 starts loading; this wave's share of tile kb's
    // scores, with tile kb-1's softmax between the MFMAs; tile kb-1's value
    // product; one barrier (tile kb+1 landed, tile kb's partial scores stored).
    auto step = [&](int kb, auto kFirst) __attribute__((always_inline)) {
      constexpr bool first = decltype(kFirst)::value;
      int lane_it = lane;
      __asm__ __volatile__("" : "+v"(lane_it));
      int32_t ahead = -1;
      if (tid < kTileKeys && kb + 2 < u.kb1)
        ahead = fetch_slot(slots_b, (kb + 2) * kTileKeys + tid, u.nkeys);
      // Tile kb+1 goes to the stage tile kb-2 used, whose value product ran
      // before the previous step's barrier.
      if (kb + 1 < u.kb1)
        issue_tile_w<DL, DR>(sm.stage[(kb + 1) % kStages], sm.slot[(kb + 1) % kRing], c_kv,
                             k_pe, wave, lane_it);
      if constexpr (first) {
        do_qk(kb, lane_it, std::false_type{});
      } else {
        do_qk(kb, lane_it, std::true_type{});
        do_pv(kb - 1, lane_it);
      }
      __builtin_amdgcn_s_waitcnt(0);  // tile kb+1 in LDS; partial scores stored
      if (tid < kTileKeys && kb + 2 < u.kb1)
        publish_slots(sm.slot[(kb + 2) % kRing], &sm.valid[(kb + 2) % kRing], ahead,
                      a.num_slots, tid);
      __syncthreads();
    };

    for (int attempt = 0;; ++attempt) {
      if (attempt > 0) {
        // The rerun: references at each row's largest score, which no tile of
        // the range exceeds.
#pragma unroll
        for (int c = 0; c < kNCBn; ++c) o[c] = f32x16_t{};
        l_run = 0.0f;
        m_ref = m_seen;
        start_tiles();
        __syncthreads();
        issue_tile_w<DL, DR>(sm.stage[u.kb0 % kStages], sm.slot[u.kb0 % kRing], c_kv, k_pe,
                             wave, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      step(u.kb0, std::true_type{});
      for (int kb = u.kb0 + 1; kb < u.kb1; ++kb) step(kb, std::false_type{});
      // Drain: the last tile's softmax and value product.
      {
        int lane_it = lane;
        __asm__ __volatile__("" : "+v"(lane_it));
        gather(u.kb1 - 1, lane_it);
#pragma unroll
        for (int j = 0; j < kParts; ++j) part(j, u.kb1 - 1, lane_it);
        do_pv(u.kb1 - 1, lane_it);
      }
      // Every wave's last value product has read the key stages before the
      // epilogue (or a rerun) writes them.
      if (!__syncthreads_or(attempt == 0 && overflow)) break;
      overflow = false;
    }
  }

  // Row sum over the two lanes of the row (the same in every wave).
  const float l = xor32_sum(l_run);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const float lse_v = l > 0.0f ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
  float* dst_lse = nullptr;
  if (u.complete) {
    if (row_exists && a.lse) dst_lse = a.lse + (long long)u.b * QH + r_loc;
  } else if (row_live) {
    dst_lse = a.ws_lse + u.slot * kRowsPerWG + rloc;
  }
  // This wave's 128 columns of the 32 rows go out through LDS (the key stages
  // are free now) in two passes of 64 columns; every store instruction writes
  // four 256-byte row segments.
  constexpr int kPCb = 2, kPCols = 32 * kPCb, kPitch = kPCols + 4;  // floats
  static_assert(kWavesW * 32 * kPitch * 4 <= kStages * G::kStageBytes, "epilogue staging");
  float* buf = reinterpret_cast<float*>(sm.stage[0]) + wave * (32 * kPitch);
  const uint32_t live_m = (uint32_t)__ballot(row_live);  // bit r: row r of the quarter
  const uint32_t exist_m = (uint32_t)__ballot(row_exists);
  const uint32_t write_m = u.complete ? exist_m : live_m;
  float* base = u.complete
                    ? a.out + ((long long)u.b * QH + (long long)u.rt * kRowsPerWG + quarter * 32) * DL
                    : a.ws_o + ((long long)u.slot * kRowsPerWG + quarter * 32) * DL;
  base += 32 * kNCBn * wave;
  const int c4 = lane & 15;
#pragma unroll
  for (int pass = 0; pass < kNCBn / kPCb; ++pass) {
#pragma unroll
    for (int c = 0; c < kPCb; ++c) {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int cb = pass * kPCb + c;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row_live)
          v = make_float4(o[cb][4 * t4] * inv, o[cb][4 * t4 + 1] * inv, o[cb][4 * t4 + 2] * inv,
                          o[cb][4 * t4 + 3] * inv);
        *reinterpret_cast<float4*>(buf + n * kPitch + c * 32 + 8 * t4 + 4 * g) = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's parked rows are in LDS
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4);
      const float4 v = *reinterpret_cast<const float4*>(buf + r * kPitch + 4 * c4);
      float* d = base + (long long)r * DL + pass * kPCols + 4 * c4;
      if ((write_m >> r) & 1u) store_through(d, v);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next pass overwrites
  }
  if (dst_lse && g == 0 && wave == 0) *dst_lse = row_live ? lse_v : -INFINITY;
  // Each wave parks its rows in its own part of stage 0, and the next unit
  // writes the stages only after the barrier of its prologue.
}

// Workgroups are placed by narrow_place (the four quarters of a range on one
// XCD); ranges past the grid (padding to whole groups of 8) have nothing to do.
template <int DL, int DR, bool kSplit2>
__global__ __launch_bounds__(kThreadsW, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void verify_attn_narrow_kernel(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ q_pe,
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe, int64_t num_slots,
    const int32_t* __restrict__ req_to_slot, int max_kv, const int32_t* __restrict__ prefix_len,
    const int32_t* __restrict__ n_nodes, const uint64_t* __restrict__ vis, int B, int Q, int H,
    int RT, float sm_scale, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, long long* __restrict__ ws_pref,
    int G) {
  __shared__ SmemN<DL, DR> sm;
  long long bl;
  int quarter;
  narrow_place(blockIdx.x, bl, quarter);
  if (bl >= (kSplit2 ? 2LL : 1LL) * G) return;
  const Args args{q_lat, q_pe, c_kv, k_pe, num_slots, req_to_slot, max_kv, vis, Q, H,
                  sm_scale * kLog2e, out, lse, ws_o, ws_lse, 0};
  for_each_unit<kThreadsW, kSplit2>(sm, prefix_len, n_nodes, B, Q, H, max_kv, RT, ws_pref, G,
                                    bl, bl == 0 && quarter == 0,
                                    [&](const Unit& u, long long) __attribute__((always_inline)) {
                                      run_unit_n<DL, DR>(sm, args, u, quarter);
                                    });
}

// Combines the partial results of row tiles whose key range was cut, and writes
// the padding output of row tiles with no live row.  Two variants share the
// contributor rule (slot 2g holds a workgroup's head unit, 2g+1 its tail) and
// read the work prefix, split mode and start cost from the workspace (the
// attention kernel's first workgroup stores them):
//  * verify_merge_kernel (few row tiles, as at batch 1): thin workgroups of
//    MergeGeo::kRows rows, so that many CUs share the work; the contributing
//    partial slots are compacted once into LDS; each
//    row's total log-sum-exp is reduced by a group of lanes; then, for batches
//    of MergeGeo::kBatch contributors, the per-(contributor, row) weights go to
//    LDS and every thread accumulates its float4 chunks with all of a batch's
//    loads independent of one another.
//  * verify_merge_wide_kernel (otherwise): see below.
template <int DL, int ROWS>
struct MergeGeo {
  static constexpr int kChunks = DL / 4;                   // float4 per row
  static constexpr int kRows = ROWS;                       // rows per workgroup
  static constexpr int kItems = kRows * kChunks / kMergeThreads;  // chunks per thread
  // Contributors whose loads are in flight at once: about 32 float4 per thread.
  static constexpr int kBatch = kItems >= 8 ? 4 : 32 / kItems > 16 ? 16 : 32 / kItems;
  static constexpr int kLanesPerRow =                      // lanes of a row's LSE
      kMergeThreads / kRows < kWave ? kMergeThreads / kRows : kWave;
  static_assert(kRows * kChunks == kMergeThreads * kItems, "merge tiling");
  static_assert(kRowsPerWG % kRows == 0 && kRows * kLanesPerRow <= kMergeThreads, "merge tiling");
};

template <int DL, int ROWS>
__global__ __launch_bounds__(kMergeThreads) void verify_merge_kernel(
    const int32_t* __restrict__ prefix_len, const int32_t* __restrict__ n_nodes, int B, int Q,
    int H, int RT, int max_kv, int grid_attn, float* __restrict__ out, float* __restrict__ lse,
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    const long long* __restrict__ ws_pref) {
  using MG = MergeGeo<DL, ROWS>;
  __shared__ int s_src[kMaxGrid];
  __shared__ int s_cnt;
  __shared__ float s_lse[MG::kRows];
  __shared__ float s_lv[MG::kBatch][MG::kRows];  // LSEs of the first batch's contributors
  __shared__ float s_w[MG::kBatch][MG::kRows];
  const int tid = threadIdx.x;
  // One workgroup per (row tile, row group), the row groups of a tile
  // consecutive; row tiles in reverse: under the aligned split the tiles to
  // merge are the last ones, and all their workgroups are dispatched before
  // those of tiles with nothing to merge.
  constexpr int kGroups = kRowsPerWG / MG::kRows;
  const int u = (int)(gridDim.x / kGroups) - 1 - (int)(blockIdx.x / kGroups);
  const int b = u / RT, rt = u % RT;
  const ReqInfo ri = req_info(prefix_len, n_nodes, b, Q, H, max_kv, RT);
  const long long QH = (long long)Q * H;
  const int r0 = (int)(blockIdx.x % kGroups) * MG::kRows;  // first row within the tile
  if ((long long)rt * kRowsPerWG + r0 >= QH) return;
  // Work prefix over requests and the split mode, as the attention kernel
  // recorded them.
  const long long Gn = grid_attn;
  const long long mode = ws_pref[B + 1];
  const int c = (int)ws_pref[B + 2];

  const bool has_work = rt < ri.vt;
  if (has_work) {
    long long S_u, Wtot, g_first, g_last;
    if (!stream_place(mode, ws_pref, B, b, rt, ri, Gn, c, S_u, Wtot)) return;  // a whole unit
    tile_owners(S_u, Wtot, Gn, ri.nkb, c, g_first, g_last);
    if (g_first == g_last) return;  // written directly by the attention kernel
    // Each contributing workgroup (non-empty range) wrote its partial for this
    // tile into slot 2g when the tile holds the start of its range, else 2g+1.
    if (tid < kWave) {
      const int cnt = (int)(g_last - g_first + 1);
      int base = 0;
      for (int k0 = 0; k0 < cnt; k0 += kWave) {
        const long long gg = g_first + k0 + tid;
        int src = -1;
        if (k0 + tid < cnt) src = (int)contributor_slot(gg, S_u, Wtot, Gn);
        const uint64_t m = __ballot(src >= 0);
        const int at = base + (int)__builtin_amdgcn_mbcnt_hi(
                                  (unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
        if (src >= 0) s_src[at] = src;
        base += __popcll(m);
      }
      if (tid == 0) s_cnt = base;
    }
  } else if (tid == 0) {
    s_cnt = 0;
  }
  __syncthreads();
  const int cnt = s_cnt;

  // The first batch's partial rows are requested before the log-sum-exps are
  // combined: they do not depend on them.
  float4 acc[MG::kItems];
  int rl_of[MG::kItems];
#pragma unroll
  for (int it = 0; it < MG::kItems; ++it) {
    acc[it] = make_float4(0.f, 0.f, 0.f, 0.f);
    rl_of[it] = (tid + it * kMergeThreads) / MG::kChunks;
  }
  const int chunk = tid % MG::kChunks;
  // Rows that no contributor wrote (not live) read stale workspace here; their
  // sums are discarded below, and every address stays inside the workspace.
  // All loads of a batch (every item, every contributor) are issued before
  // the first is used.
  float4 v[MG::kItems][MG::kBatch];
  auto load_batch = [&](int k0, int nk) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < MG::kItems; ++it) {
#pragma unroll
      for (int k = 0; k < MG::kBatch; ++k) {
        if (k < nk) {
          const float* src =
              ws_o + ((long long)s_src[k0 + k] * kRowsPerWG + r0 + rl_of[it]) * DL + chunk * 4;
          v[it][k] = *reinterpret_cast<const float4*>(src);
        }
      }
    }
  };
  load_batch(0, cnt < MG::kBatch ? cnt : MG::kBatch);

  // Row log-sum-exp: kLanesPerRow lanes per row, each over every
  // kLanesPerRow-th contributor, then a butterfly over the group.
  if (tid < MG::kRows * MG::kLanesPerRow) {
    const int rl = tid / MG::kLanesPerRow, j = tid % MG::kLanesPerRow;
    const int rr = r0 + rl;
    const long long r_loc = (long long)rt * kRowsPerWG + rr;
    const bool live = r_loc < QH && (int)(r_loc / H) < ri.nb;
    float m = -INFINITY, z = 0.0f;
    if (live) {
      for (int k = j; k < cnt; k += MG::kLanesPerRow) {
        const float x = ws_lse[(long long)s_src[k] * kRowsPerWG + rr];
        if (k < MG::kBatch) s_lv[k][rl] = x;
        if (x == -INFINITY) continue;
        if (x > m) {
          z = z * __expf(m - x) + 1.0f;
          m = x;
        } else {
          z += __expf(x - m);
        }
      }
    }
#pragma unroll
    for (int off = 1; off < MG::kLanesPerRow; off <<= 1) {
      const float m2 = __shfl_xor(m, off), z2 = __shfl_xor(z, off);
      const float mn = fmaxf(m, m2);
      if (mn != -INFINITY) {
        z = (m == -INFINITY ? 0.0f : z * __expf(m - mn)) +
            (m2 == -INFINITY ? 0.0f : z2 * __expf(m2 - mn));
        m = mn;
      }
    }
    if (j == 0) s_lse[rl] = z > 0.0f ? m + __logf(z) : -INFINITY;
  }
  __syncthreads();

  for (int k0 = 0; k0 < cnt; k0 += MG::kBatch) {
    const int nk = cnt - k0 < MG::kBatch ? cnt - k0 : MG::kBatch;
    if (k0 > 0) load_batch(k0, nk);
    for (int e = tid; e < MG::kBatch * MG::kRows; e += kMergeThreads) {
      const int k = e / MG::kRows, rl = e % MG::kRows;
      const float lt = s_lse[rl];
      float w = 0.0f;
      if (k < nk && lt != -INFINITY) {
        const float x = k0 == 0 ? s_lv[k][rl]
                                : ws_lse[(long long)s_src[k0 + k] * kRowsPerWG + r0 + rl];
        if (x != -INFINITY) w = __expf(x - lt);
      }
      s_w[k][rl] = w;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < MG::kItems; ++it) {
#pragma unroll
      for (int k = 0; k < MG::kBatch; ++k) {
        if (k < nk) {
          const float w = s_w[k][rl_of[it]];
          acc[it].x = __builtin_fmaf(w, v[it][k].x, acc[it].x);
          acc[it].y = __builtin_fmaf(w, v[it][k].y, acc[it].y);
          acc[it].z = __builtin_fmaf(w, v[it][k].z, acc[it].z);
          acc[it].w = __builtin_fmaf(w, v[it][k].w, acc[it].w);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int it = 0; it < MG::kItems; ++it) {
    const long long r_loc = (long long)rt * kRowsPerWG + r0 + rl_of[it];
    if (r_loc >= QH) continue;
    const long long grow = (long long)b * QH + r_loc;
    const float lt = s_lse[rl_of[it]];
    *reinterpret_cast<float4*>(out + grow * DL + chunk * 4) =
        lt != -INFINITY ? acc[it] : make_float4(0.f, 0.f, 0.f, 0.f);
    if (lse && chunk == 0) lse[grow] = lt;
  }
}

// The merge for many row tiles: 8 rows of 512 (16 of 64) per workgroup.  The
// first kMergePreW contributors'
// partial rows are requested before the row log-sum-exps are reduced (they do
// not depend on them), and the log-sum-exps read for that reduction are kept
// in LDS for the weights, so the bulk of the reads starts one dependent round
// trip after the contributor list.
template <int DL>
struct MergeGeoW {
  static constexpr int kChunks = DL / 4;                          // float4 per row
  static constexpr int kItems = DL >= 256 ? 4 : 1;                // chunks per thread
  static constexpr int kRows = kMergeThreads * kItems / kChunks;  // rows per workgroup
  static constexpr int kLanesPerRow = kMergeThreads / kRows;      // lanes of a row's LSE
  static_assert(kRows * kChunks == kMergeThreads * kItems, "merge tiling");
  static_assert(kRowsPerWG % kRows == 0 && kLanesPerRow <= kWave, "merge tiling");
};
constexpr int kMergeBatchW = 32;  // contributors whose weights are staged at once

constexpr int kMergePreW = 3;     // contributors whose rows are requested up front

template <int DL>
__global__ __launch_bounds__(kMergeThreads) void verify_merge_wide_kernel(
    const int32_t* __restrict__ prefix_len, const int32_t* __restrict__ n_nodes, int B, int Q,
    int H, int RT, int max_kv, int grid_attn, float* __restrict__ out, float* __restrict__ lse,
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    const long long* __restrict__ ws_pref) {
  using MG = MergeGeoW<DL>;
  __shared__ int s_src[kMaxGrid];
  __shared__ int s_cnt;
  __shared__ float s_lse[MG::kRows];
  __shared__ float s_lv[kMergeBatchW][MG::kRows];  // LSEs of the first batch's contributors
  __shared__ float s_w[kMergeBatchW][MG::kRows];
  // The stream prefix, split mode and start cost the attention kernel
  // recorded.
  const long long mode = ws_pref[B + 1];
  const int c = (int)ws_pref[B + 2];
  // Under the aligned split every request has the same row-tile count vt0 =
  // mode / B, and units b * vt0 + rt below q * G are whole (written by the
  // attention kernel): such items are skipped without reading the request.
  const long long q_whole = mode >= 0 ? (mode / grid_attn) * grid_attn : 0;
  const int vt0 = mode >= 0 ? (int)(mode / B) : 0;
  // One work item per (row tile, row group), the row groups of a tile
  // consecutive and the row tiles in reverse: under the aligned split the
  // tiles to merge are the last ones.  The grid holds at most the workgroups
  // the chip keeps resident, each taking every gridDim.x-th item, so that
  // items with nothing to merge (whole units under the aligned split) cost a
  // few instructions instead of a dispatch.
  constexpr int kGroups = kRowsPerWG / MG::kRows;
  const int units = B * RT;
  auto item = [&](int i) __attribute__((always_inline)) {
    // The thread index through an empty asm, so that per-thread values are
    // formed inside each item rather than hoisted and held across the loop.
    int tid = threadIdx.x;
    __asm__ __volatile__("" : "+v"(tid));
    const int u = units - 1 - i / kGroups;
    const int b = u / RT, rt = u % RT;
    const long long QH = (long long)Q * H;
    const int r0 = (i % kGroups) * MG::kRows;  // first row within the tile
    if ((long long)rt * kRowsPerWG + r0 >= QH) return;
    if (rt < vt0 && (long long)b * vt0 + rt < q_whole) return;
    const ReqInfo ri = req_info(prefix_len, n_nodes, b, Q, H, max_kv, RT);
    const long long Gn = grid_attn;

    const bool has_work = rt < ri.vt;
    if (has_work) {
      long long S_u, Wtot, g_first, g_last;
      if (!stream_place(mode, ws_pref, B, b, rt, ri, Gn, c, S_u, Wtot)) return;  // a whole unit
      tile_owners(S_u, Wtot, Gn, ri.nkb, c, g_first, g_last);
      if (g_first == g_last) return;  // written directly by the attention kernel
      // Each contributing workgroup (non-empty range) wrote its partial for this
      // tile into slot 2g when the tile holds the start of its range, else 2g+1.
      if (tid < kWave) {
        const int cnt = (int)(g_last - g_first + 1);
        int base = 0;
        for (int k0 = 0; k0 < cnt; k0 += kWave) {
          const long long gg = g_first + k0 + tid;
          int src = -1;
          if (k0 + tid < cnt) src = (int)contributor_slot(gg, S_u, Wtot, Gn);
          const uint64_t m = __ballot(src >= 0);
          const int at = base + (int)__builtin_amdgcn_mbcnt_hi(
                                    (unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
          if (src >= 0) s_src[at] = src;
          base += __popcll(m);
        }
        if (tid == 0) s_cnt = base;
      }
    } else if (tid == 0) {
      s_cnt = 0;
    }
    __syncthreads();
    const int cnt = s_cnt;

    // Rows of this thread's chunks and the first kMergePreW contributors' partial
    // rows, requested now.  Rows that no contributor wrote (not live) read stale
    // workspace; their sums are discarded below, and every address stays inside
    // the workspace.
    float4 acc[MG::kItems];
    int rl_of[MG::kItems];
#pragma unroll
    for (int it = 0; it < MG::kItems; ++it) {
      acc[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      rl_of[it] = (tid + it * kMergeThreads) / MG::kChunks;
    }
    const int chunk = tid % MG::kChunks;
    const int npre = cnt < kMergePreW ? cnt : kMergePreW;
    float4 pre[kMergePreW][MG::kItems];
#pragma unroll
    for (int k = 0; k < kMergePreW; ++k) {
#pragma unroll
      for (int it = 0; it < MG::kItems; ++it) pre[k][it] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k < npre) {
        const float* src = ws_o + ((long long)s_src[k] * kRowsPerWG + r0) * DL + chunk * 4;
#pragma unroll
        for (int it = 0; it < MG::kItems; ++it)
          pre[k][it] = *reinterpret_cast<const float4*>(src + (long long)rl_of[it] * DL);
      }
    }

    // Row log-sum-exp: kLanesPerRow lanes per row, each over every
    // kLanesPerRow-th contributor (keeping the first batch's values in LDS),
    // then a butterfly over the group.
    {
      const int rl = tid / MG::kLanesPerRow, j = tid % MG::kLanesPerRow;
      const int rr = r0 + rl;
      const long long r_loc = (long long)rt * kRowsPerWG + rr;
      const bool live = r_loc < QH && (int)(r_loc / H) < ri.nb;
      float m = -INFINITY, z = 0.0f;
      for (int k = j; k < kMergeBatchW; k += MG::kLanesPerRow) s_lv[k][rl] = -INFINITY;
      if (live) {
        for (int k = j; k < cnt; k += MG::kLanesPerRow) {
          const float v = ws_lse[(long long)s_src[k] * kRowsPerWG + rr];
          if (k < kMergeBatchW) s_lv[k][rl] = v;
          if (v == -INFINITY) continue;
          if (v > m) {
            z = z * __expf(m - v) + 1.0f;
            m = v;
          } else {
            z += __expf(v - m);
          }
        }
      }
#pragma unroll
      for (int off = 1; off < MG::kLanesPerRow; off <<= 1) {
        const float m2 = __shfl_xor(m, off), z2 = __shfl_xor(z, off);
        const float mn = fmaxf(m, m2);
        if (mn != -INFINITY) {
          z = (m == -INFINITY ? 0.0f : z * __expf(m - mn)) +
              (m2 == -INFINITY ? 0.0f : z2 * __expf(m2 - mn));
          m = mn;
        }
      }
      if (j == 0) s_lse[rl] = z > 0.0f ? m + __logf(z) : -INFINITY;
    }
    __syncthreads();

    for (int k0 = 0; k0 < cnt; k0 += kMergeBatchW) {
      const int nk = cnt - k0 < kMergeBatchW ? cnt - k0 : kMergeBatchW;
      for (int e = tid; e < kMergeBatchW * MG::kRows; e += kMergeThreads) {
        const int k = e / MG::kRows, rl = e % MG::kRows;
        const float lt = s_lse[rl];
        float w = 0.0f;
        if (k < nk && lt != -INFINITY) {
          const float v = k0 == 0 ? s_lv[k][rl]
                                  : ws_lse[(long long)s_src[k0 + k] * kRowsPerWG + r0 + rl];
          if (v != -INFINITY) w = __expf(v - lt);
        }
        s_w[k][rl] = w;
      }
      __syncthreads();
      if (k0 == 0) {
#pragma unroll
        for (int k = 0; k < kMergePreW; ++k) {
          if (k >= npre) break;
#pragma unroll
          for (int it = 0; it < MG::kItems; ++it) {
            const float w = s_w[k][rl_of[it]];
            acc[it].x = __builtin_fmaf(w, pre[k][it].x, acc[it].x);
            acc[it].y = __builtin_fmaf(w, pre[k][it].y, acc[it].y);
            acc[it].z = __builtin_fmaf(w, pre[k][it].z, acc[it].z);
            acc[it].w = __builtin_fmaf(w, pre[k][it].w, acc[it].w);
          }
        }
      }
#pragma unroll 8
      for (int k = k0 == 0 ? npre : 0; k < nk; ++k) {
        const float* src = ws_o + ((long long)s_src[k0 + k] * kRowsPerWG + r0) * DL + chunk * 4;
#pragma unroll
        for (int it = 0; it < MG::kItems; ++it) {
          const float w = s_w[k][rl_of[it]];
          const float4 v = *reinterpret_cast<const float4*>(src + (long long)rl_of[it] * DL);
          acc[it].x = __builtin_fmaf(w, v.x, acc[it].x);
          acc[it].y = __builtin_fmaf(w, v.y, acc[it].y);
          acc[it].z = __builtin_fmaf(w, v.z, acc[it].z);
          acc[it].w = __builtin_fmaf(w, v.w, acc[it].w);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int it = 0; it < MG::kItems; ++it) {
      const long long r_loc = (long long)rt * kRowsPerWG + r0 + rl_of[it];
      if (r_loc >= QH) continue;
      const long long grow = (long long)b * QH + r_loc;
      const float lt = s_lse[rl_of[it]];
      *reinterpret_cast<float4*>(out + grow * DL + chunk * 4) =
          lt != -INFINITY ? acc[it] : make_float4(0.f, 0.f, 0.f, 0.f);
      if (lse && chunk == 0) lse[grow] = lt;
    }
    __syncthreads();  // the next item rewrites the LDS this one read
  };
#pragma unroll 1
  for (int i = blockIdx.x; i < units * kGroups; i += gridDim.x) item(i);
}

// Workgroups of the wide merge: all its items, or as many as the chip keeps
// resident at once (from the compiled kernel's occupancy), whichever is fewer.
template <int DL>
int merge_wide_grid(int items, int num_cu) {
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, verify_merge_wide_kernel<DL>,
                                                     kMergeThreads, 0) != hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  const long long resident = (long long)per_cu * (num_cu > 0 ? num_cu : 256);
  return items < resident ? items : (int)resident;
}

// Polls of a pair wait before it gives up.  DDT_PAIR_SPIN_LIMIT (read once)
// lowers it, so that a test can make every wait give up at once and check
// that the rows come out as NaN; every wait still ends.
int pair_spin_limit() {
  static const int v = [] {
    const char* e = getenv("DDT_PAIR_SPIN_LIMIT");
    if (!e || !*e) return kSpinLimit;
    const long x = strtol(e, nullptr, 10);
    return x < 0 ? 0 : (x > kSpinLimit ? kSpinLimit : (int)x);
  }();
  return v;
}

template <typename T, int DL, int DR>
hipError_t launch_impl(const void* q_lat, const void* q_pe, const void* c_kv, const void* k_pe,
                       int64_t num_slots, const int32_t* req_to_slot, int max_kv,
                       const int32_t* prefix_len, const int32_t* n_nodes, const uint64_t* vis,
                       int B, int Q, int H, float sm_scale, float* out, float* lse,
                       void* workspace, const AttnPlan& plan, hipStream_t stream,
                       int phases) {
  float* ws_o = static_cast<float*>(workspace);
  float* ws_lse = ws_o + (size_t)2 * plan.grid * kRowsPerWG * DL;
  long long* ws_pref = reinterpret_cast<long long*>(ws_lse + (size_t)2 * plan.grid * kRowsPerWG);
  // Twice the workgroups, and the kernel that can take the aligned split, when
  // that split can apply (B * row tiles >= G); the kernel decides from the data
  // whether it does.
  const bool split2 = (long long)B * plan.row_tiles >= plan.grid;
  if (!(phases & kPhaseAttention)) {
  } else if constexpr (Geo<T, DL, DR>::kBF16 && DL == 512 && DR == 64) {
    if (plan.narrow) {
      // Four workgroups per range, the ranges padded to whole groups of 8
      // (one per XCD).
      const long long blocks = narrow_blocks(split2 ? 2LL * plan.grid : (long long)plan.grid);
      auto kernel = split2 ? verify_attn_narrow_kernel<DL, DR, true>
                           : verify_attn_narrow_kernel<DL, DR, false>;
      hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreadsW), 0, stream,
                         static_cast<const T*>(q_lat), static_cast<const T*>(q_pe),
                         static_cast<const T*>(c_kv), static_cast<const T*>(k_pe), num_slots,
                         req_to_slot, max_kv, prefix_len, n_nodes, vis, B, Q, H, plan.row_tiles,
                         sm_scale, out, lse, ws_o, ws_lse, ws_pref, plan.grid);
    } else {
    auto kernel = split2 ? verify_attn_wide_kernel<DL, DR, true>
                         : verify_attn_wide_kernel<DL, DR, false>;
    hipLaunchKernelGGL(kernel, dim3(split2 ? 2 * plan.grid : plan.grid), dim3(kThreadsW), 0,
                       stream, static_cast<const T*>(q_lat), static_cast<const T*>(q_pe),
                       static_cast<const T*>(c_kv), static_cast<const T*>(k_pe), num_slots,
                       req_to_slot, max_kv, prefix_len, n_nodes, vis, B, Q, H, plan.row_tiles,
                       sm_scale, out, lse, ws_o, ws_lse, ws_pref, plan.grid);
    }
  } else {
    auto kernel =
        split2 ? verify_attn_kernel<T, DL, DR, true> : verify_attn_kernel<T, DL, DR, false>;
    hipLaunchKernelGGL(kernel, dim3(split2 ? 2 * plan.grid : plan.grid), dim3(kThreads), 0,
                       stream, static_cast<const T*>(q_lat), static_cast<const T*>(q_pe),
                       static_cast<const T*>(c_kv), static_cast<const T*>(k_pe), num_slots,
                       req_to_slot, max_kv, prefix_len, n_nodes, vis, B, Q, H, plan.row_tiles,
                       sm_scale, out, lse, ws_o, ws_lse, ws_pref, plan.grid, pair_spin_limit());
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !(phases & kPhaseMerge)) return e;
  // Thin merge workgroups (2 rows of 512) when there are so few row tiles that
  // the wide merge would leave most CUs idle.
  const int units = B * plan.row_tiles;
  constexpr int kRn = MergeGeoW<DL>::kRows, kRs = DL >= 256 ? 2 : 16;
  if (units * (kRowsPerWG / kRn) < plan.num_cu)
    hipLaunchKernelGGL((verify_merge_kernel<DL, kRs>), dim3(units * (kRowsPerWG / kRs)),
                       dim3(kMergeThreads), 0, stream, prefix_len, n_nodes, B, Q, H,
                       plan.row_tiles, max_kv, plan.grid, out, lse, ws_o, ws_lse, ws_pref);
  else
    hipLaunchKernelGGL((verify_merge_wide_kernel<DL>),
                       dim3(merge_wide_grid<DL>(units * (kRowsPerWG / kRn), plan.num_cu)),
                       dim3(kMergeThreads), 0,
                       stream, prefix_len, n_nodes, B, Q, H, plan.row_tiles, max_kv, plan.grid,
                       out, lse, ws_o, ws_lse, ws_pref);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_attn(int dtype, int d_lat, int d_rope, const void* q_lat,
                              const void* q_pe, const void* c_kv, const void* k_pe,
                              int64_t num_slots, const int32_t* req_to_slot, int max_kv,
                              const int32_t* prefix_len, const int32_t* n_nodes,
                              const uint64_t* vis, int B, int Q, int H, float sm_scale,
                              float* out, float* lse, void* workspace, const AttnPlan& plan,
                              hipStream_t stream, int phases) {
  // dtype: 0 = f32, 1 = bf16 (validated by the caller).
  if (dtype == 1 && d_lat == 512 && d_rope == 64)
    return launch_impl<uint16_t, 512, 64>(q_lat, q_pe, c_kv, k_pe, num_slots, req_to_slot,
                                          max_kv, prefix_len, n_nodes, vis, B, Q, H, sm_scale,
                                          out, lse, workspace, plan, stream, phases);
  if (dtype == 1 && d_lat == 64 && d_rope == 16)
    return launch_impl<uint16_t, 64, 16>(q_lat, q_pe, c_kv, k_pe, num_slots, req_to_slot,
                                         max_kv, prefix_len, n_nodes, vis, B, Q, H, sm_scale,
                                         out, lse, workspace, plan, stream, phases);
  if (dtype == 0 && d_lat == 64 && d_rope == 16)
    return launch_impl<float, 64, 16>(q_lat, q_pe, c_kv, k_pe, num_slots, req_to_slot, max_kv,
                                      prefix_len, n_nodes, vis, B, Q, H, sm_scale, out, lse,
                                      workspace, plan, stream, phases);
  return hipErrorInvalidValue;
}

}  // namespace ddt
