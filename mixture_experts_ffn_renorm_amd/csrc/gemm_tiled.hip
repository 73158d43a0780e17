// LDS-tiled MFMA grouped GEMMs for batches with many pairs per expert.
//
// GEMM 1 (page "Mixture of Experts in vLLM - From First Principles to
// fused_moe", sub-section "One GEMM 1 program, step by step"): a tile is one
// block of BM pairs (one expert, from the index lists) and 128 columns of
// the activation.  It reads expert_ids[b], skips pad entries
// (id >= M*top_k), reads input row p // top_k of x in place, multiplies by
// the matching 128 gate rows and 128 up rows of W13[e], and writes
// SiLU(gate) * up to row p of act (sub-section "The rest of the layer stays
// in pair order"), so the [M*top_k, 2I] product never reaches memory.
//
// GEMM 2 (same page, "The rest of the layer stays in pair order"): the same
// tiling over act (row p read directly) and 256 rows of W2[e]; row p of the
// bf16 pair-order product [M*top_k, H] is written in place (the page's
// cache3).  A second small kernel reads, per token, its top_k rows and adds
// them weighted by topk_weights in slot order (section "Put the results
// back, and combine them per token": moe_sum with the routed weights).
//
// Tile: 256 weight rows x BM pairs (BM = 64, 128 or 256) x 64 k per stage,
// 8 waves in a 4 x 2 layout, each wave 64 weight rows x BM/2 pairs of
// 16x16x32 bf16 MFMAs.  Weights are the MFMA A operand and pairs the B
// operand, so each lane ends with 4 consecutive features of one pair.  With
// BM = 256 an expert of up to 256 pairs reads each weight tile once, and
// each k step of LDS operands feeds twice the MFMAs of BM = 128 (measured:
// about 1.3x the rate).  Quarters of the block that hold only pads (the
// tail of an expert's last block) skip their MFMAs.
//
// Copy waves (bf16 tiles): each workgroup has four more waves, one per
// SIMD, that issue every global-to-LDS copy and do no MFMA work, and the
// eight MFMA waves issue no copies.  The per-CU copy path drains a 64 KB
// stage far slower than waves can issue it, so a copy instruction blocks
// its wave at issue; with the copies in their own waves that block never
// holds up an MFMA (the MFMA waves spent a third of their time there).
// Copy and MFMA waves run separate loops over the same barriers, so
// neither keeps the other's registers live (104 VGPRs at 128 pairs, 168 at
// 256, for 12 waves a CU).  MXFP8 tiles take the same form at 128 pairs
// (each copy wave also copies the scale bytes of two 64-row groups).
//
// Persistent workgroups, one per CU.  Each XCD owns a contiguous range of
// tiles (block-major, all column tiles of a block side by side) and its
// workgroups take them round robin, so the column tiles of one block (same
// gathered rows) and the same column tile of an expert's adjacent blocks
// (same weights) run together under one L2.  A workgroup streams its whole
// sequence of (tile, k-step) stages through one LDS ring (3 stages; 2 of
// 64 KB for BM = 256): the loads of the next tile start while the current
// one finishes and runs its epilogue.  A tile's pair ids and expert id are
// copied into LDS by the same asynchronous copies two tiles ahead.
//
// MXFP8 operands (kMX; OCP microscaling: E4M3 bytes, one E8M0 scale per 32
// consecutive k): the same 128-byte row pieces, now 128 k values each, so a
// stage is one k step of the gfx950 scaled MFMA 16x16x128.  That MFMA reads
// from lane (r, g) the 16 bytes at k 16g .. 16g + 15 and the 16 bytes at
// 64 + 16g .. (measured with in-bounds probes: byte i of lane group g sits
// at k 64 (i / 16) + 16 g + i % 16, E4M3 as OCP defines it), which are
// exactly the two 16-byte chunks g and 4 + g the bf16 form reads for its
// two k halves, and takes the scale of k block s (32 values) of row r from
// lane r + 16 s.  Each stage also copies 4 scale bytes per row (the stage's
// four blocks) into an LDS area after the operands, one 4-byte copy per
// lane: 512 rows, the ones past the tile reading the zeroed page.
//
// Copies go from global memory straight into LDS with
// global_load_lds_dwordx4 (no register staging).  One copy instruction of a
// wave fills 1 KB of LDS = 8 rows of 64 k values; a row's eight 16-byte
// chunks are stored XOR-swizzled (chunk c of row R at slot c ^ ((R >> 1) &
// 7)), so the 16 rows that one MFMA operand read touches fall on distinct
// banks, while each global access still reads whole 128-byte row pieces.
// Rows or k ranges outside the operands (pads, features past the end, the K
// tail) copy a zeroed 16-byte page.
#include <algorithm>
#include <type_traits>

#include "moe_common.h"

using namespace moe;

namespace {

constexpr int kBK = 64;          // k elements per stage = 128 bytes per row
constexpr int kWaves = 8;
constexpr int kRowBytes = kBK * 2;
// Tile metadata buffers (pair ids, expert).  Tile i + 3's copies start when
// the copy sources of tile i are set up, up to three stages before tile i's
// first stage; the buffer they overwrite, tile i - 4's, has had its last
// stage (at most four stages before) and epilogue by then.
constexpr int kMeta = 7;

// Tile shape per block size BM: 256 weight rows x BM pairs, MFMA waves in a
// 4 (features, 64 rows each) x 2 (pair halves) layout.  With kPC four more
// waves (one per SIMD) issue every copy and the eight MFMA waves issue
// none, so a copy that blocks at issue never holds up an MFMA.
template <int BM, bool kMX = false, bool kPC = false>
struct TileCfg {
  static constexpr int kBN = 256;                      // weight rows per tile
  static constexpr int kWF = kBN / 64;
  static constexpr int kWP = kWaves / kWF;
  static constexpr int kCopyWaves = kPC ? 4 : kWaves;  // waves that issue copies
  static constexpr int kThreadsT = (kWaves + (kPC ? 4 : 0)) * 64;
  static constexpr int kWGroups = kBN / 8 / kCopyWaves;   // 8-row W groups per copy wave
  static constexpr int kXGroups = BM / 8 / kCopyWaves;    // 8-row X groups per copy wave
  // copy instructions per stage (MX: one more, the scales)
  // MX: the scale bytes of 512 rows per stage, 64 rows per 4-byte copy
  static constexpr int kScaleCopies = kMX ? kWaves / kCopyWaves : 0;
  static constexpr int kLoads = kWGroups + kXGroups + kScaleCopies;
  static constexpr int kOperandBytes = (kBN + BM) * kRowBytes;       // 40, 48 or 64 KB
  static constexpr int kScaleRows = kWaves * 64;                     // MX: 4 bytes each
  static constexpr int kStageBytes = kOperandBytes + (kMX ? kScaleRows * 4 : 0);
  static constexpr int kStages = BM == 256 ? 2 : 3;    // ring within 160 KB of LDS
  static constexpr int kRingBytes = kStages * kStageBytes;
  static constexpr int kNT = BM / kWP / 16;           // 16-pair MFMA tiles per wave
};

// Slot of a row's 16-byte chunk: chunk c of row R sits at c ^ swz(R).  With
// this choice the 16 rows read by one MFMA operand load (same chunk, rows
// R0..R0+15) hit distinct LDS banks on gfx950 (measured: the same
// ds_read_b128 throughput as contiguous reads; a 144-byte padded row
// stride, or the XOR with (R ^ (R >> 3)) & 7, both run at about half).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8 cat_u32x4(u32x4 lo, u32x4 hi) {
  const u32x4 l = lo, h = hi;   // by value
  return i32x8{(int)l[0], (int)l[1], (int)l[2], (int)l[3], (int)h[0], (int)h[1], (int)h[2], (int)h[3]};
}

// D = A B + C over 128 k of E4M3 operands, each lane's 32 values scaled by
// 2^(its E8M0 byte - 127) (format code 0 = E4M3 for both operands).
__device__ __forceinline__ f32x4 mfma_mx_16x16x128(i32x8 a, i32x8 b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Each active lane copies 4 bytes from src to LDS at lds_dst + 4 * lane.
__device__ __forceinline__ void load_lds4(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)lds_dst, 4, 0, 0);
}

struct TileParams {
  const uint16_t* a_src;   // GEMM 1: x [M, H]; GEMM 2: act [P, I]  (MX: E4M3 bytes)
  const uint16_t* w;       // GEMM 1: w13 [E, 2I, H]; GEMM 2: w2 [E, H, I]
  const uint8_t* a_scales; // MX: E8M0 per 32 k of each a_src row
  const uint8_t* w_scales; // MX: E8M0 per 32 k of each weight row
  const int32_t* sorted;
  const int32_t* expert_ids;
  const int32_t* boff;
  int M, top_k, E, H, I;
  int ntn;                 // column tiles per block
  uint16_t* out;           // GEMM 1: act [P, I]; GEMM 2: pair-order product [P, H]
  // group-quantized weights (QB = 4 or 8): codes [rows, K*QB/8], bf16 scales
  // and biases [rows, K/64]
  const uint8_t* wq;
  const uint8_t* wsc;
  const uint8_t* wbi;
};

// QB = 4 or 8: the weights are group-quantized codes (copy-wave tiles,
// BM = 128 only, 16 waves: four more widen the codes into bf16 weight
// tiles); see the quantized ring below.
template <int BM, bool kGemm1, bool kMX, bool kPC = false, int QB = 0>
__global__ __launch_bounds__((QB > 0 ? 1024 : TileCfg<BM, kMX, kPC>::kThreadsT), 1) void gemm_tiled_kernel(
    const TileParams prm) {
  using C = TileCfg<BM, kMX, kPC>;
  static_assert(QB == 0 || (kPC && !kMX && BM == 128), "quantized tiles: copy waves, 128 pairs");
  constexpr int NT = C::kNT;
  constexpr int kStages = C::kStages;
  constexpr int kBN = C::kBN;
  constexpr int kHalf = kBN / 2;   // GEMM 1: gate rows, then as many up rows
  // Quantized ring (QB > 0): two A slots hold a stage's widened bf16 weight
  // rows, kQXD + 1 B slots the gathered pair rows, three code slots the
  // stage's packed codes (kBN rows x 64 * QB / 8 bytes) and three scale
  // slots one 32-bit word of the scales, then of the biases, per weight row.
  constexpr int kQASlot = kBN * kRowBytes;                      // 32 KB
  constexpr int kQBSlot = BM * kRowBytes;                       // 16 KB
  constexpr int kQCB = kBK * (QB > 0 ? QB : 8) / 8;             // code bytes per row and stage
  constexpr int kQCSlot = kBN * kQCB;                           // 8 / 16 KB
  constexpr int kQSSlot = kBN * 4 * 2;                          // 2 KB
  // pair rows are copied kQXD stages ahead into kQXD + 1 B slots (8 bits:
  // one, so that three 16 KB code slots fit in LDS)
  constexpr int kQXD = QB == 8 ? 1 : 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  __shared__ __attribute__((aligned(16))) int s_pair[kMeta][BM];
  __shared__ int s_exp[kMeta];

  const int P = prm.M * prm.top_k;
  const int Ke = kGemm1 ? prm.H : prm.I;   // k elements
  const int K = kMX ? Ke / 2 : Ke;          // k in 2-byte units (MX: Ke % 128 == 0)
  const int ntn = prm.ntn;
  const int njobs = prm.boff[prm.E] * ntn;
  // tiles of this workgroup: j0, j0 + nslots, ... inside its XCD's range
  const int xcd = blockIdx.x & 7, nslots = gridDim.x >> 3, myslot = blockIdx.x >> 3;
  const int chunk = ceil_div(njobs, 8);
  const int j0 = xcd * chunk + myslot;
  const int jend = min(njobs, (xcd + 1) * chunk);
  if (j0 >= jend) return;   // whole workgroup
  const int nmine = ceil_div(jend - j0, nslots);
  const int nk = ceil_div(K, kBK);
  const int G = nmine * nk;  // stages of this workgroup
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int lrow = lane >> 3, lpos = lane & 7;
  // copy wave index (kPC: waves kWaves.. copy, waves 0..kWaves-1 multiply)
  // QB > 0: waves kWaves + 4 .. kWaves + 7 widen the quantized weights
  const bool widener = QB > 0 && wv >= kWaves + 4;
  const bool copier = (!kPC || wv >= kWaves) && !widener;
  const int cw = kPC ? wv - kWaves - (widener ? 4 : 0) : wv;

  // ---- metadata copies of tile i into buffer i % kMeta ----
  auto issue_meta = [&](int i) {
    if (i >= nmine) return;
    const int b = (j0 + i * nslots) / ntn;
    if (copier && cw == 0 && lane < BM / 4)
      load_lds16(prm.sorted + (size_t)b * BM + 4 * lane, reinterpret_cast<uint8_t*>(s_pair[i % kMeta]));
    if (copier && cw == 1 && lane == 0) load_lds4(prm.expert_ids + b, &s_exp[i % kMeta]);
  };

  // ---- per-lane copy sources of the tile being issued ----
  // src: the next 16 bytes this lane copies; step: elements to advance per
  // stage (0 for rows outside the operands, which read the zeroed page).
  // Only the last stage of a K with a tail checks k against K.
  const uint16_t* wsrc[C::kWGroups];
  const uint16_t* xsrc[C::kXGroups];
  int wstep[C::kWGroups], xstep[C::kXGroups];
  const uint16_t* zero = reinterpret_cast<const uint16_t*>(kZeroPage);
  const bool k_tail = (K % kBK) != 0;
  // MX: this lane copies the 4 scale bytes of rows 64 (cw + kCopyWaves h) +
  // lane of the tile (weight rows, then pair rows, then unused) per stage
  const uint8_t* ssrc[C::kScaleCopies > 0 ? C::kScaleCopies : 1];
  int sstep[C::kScaleCopies > 0 ? C::kScaleCopies : 1];

  // Point the pair-row copy sources at tile i (its metadata is in LDS).
  auto setup_x = [&](int i) {
    const int buf = i % kMeta;
#pragma unroll
    for (int gi = 0; gi < C::kXGroups; ++gi) {
      const int R = (cw + C::kCopyWaves * gi) * 8 + lrow;
      const int p = s_pair[buf][R];
      const uint16_t* row = nullptr;
      if (p < P)
        row = kGemm1 ? prm.a_src + (size_t)(p / prm.top_k) * K    // K: row length in
                     : prm.a_src + (size_t)p * K;                 // 2-byte units
      xsrc[gi] = row != nullptr ? row + (lpos ^ swz(R)) * 8 : zero;
      xstep[gi] = row != nullptr ? kBK : 0;
    }
  };

  // Point the copy sources at tile i (its metadata is in LDS), and start the
  // metadata copies of tile i + 3.
  auto setup = [&](int i) {
    const int buf = i % kMeta;
    const int j = j0 + i * nslots;
    const int nt = j - (j / ntn) * ntn;
    const int e = s_exp[buf];
#pragma unroll
    for (int gi = 0; gi < C::kWGroups; ++gi) {
      const int R = (cw + C::kCopyWaves * gi) * 8 + lrow;
      const uint16_t* row = nullptr;
      if (kGemm1) {
        const int f = nt * kHalf + (R % kHalf);
        if (f < prm.I)
          row = prm.w + ((size_t)e * 2 * prm.I + (R < kHalf ? f : prm.I + f)) * K;
      } else {
        const int h = nt * kBN + R;
        if (h < prm.H) row = prm.w + ((size_t)e * prm.H + h) * K;
      }
      wsrc[gi] = row != nullptr ? row + (lpos ^ swz(R)) * 8 : zero;
      wstep[gi] = row != nullptr ? kBK : 0;
    }
    setup_x(i);
#pragma unroll
    for (int h = 0; h < C::kScaleCopies; ++h) {
      const int R = (cw + C::kCopyWaves * h) * 64 + lane, nb = Ke / 32;
      const uint8_t* srow = nullptr;
      if (R < kBN) {
        if (kGemm1) {
          const int f = nt * kHalf + (R % kHalf);
          if (f < prm.I)
            srow = prm.w_scales + ((size_t)e * 2 * prm.I + (R < kHalf ? f : prm.I + f)) * nb;
        } else {
          const int h = nt * kBN + R;
          if (h < prm.H) srow = prm.w_scales + ((size_t)e * prm.H + h) * nb;
        }
      } else if (R < kBN + BM) {
        const int p = s_pair[buf][R - kBN];
        if (p < P)
          srow = prm.a_scales + (size_t)(kGemm1 ? p / prm.top_k : p) * nb;
      }
      ssrc[h] = srow != nullptr ? srow : reinterpret_cast<const uint8_t*>(kZeroPage);
      sstep[h] = srow != nullptr ? 4 : 0;
    }
    issue_meta(i + 3);
  };

  int is_i = 0, is_kt = 0, is_slot = 0;
  auto issue_stage = [&]() {
    const int kt = is_kt;
    if (kt == 0) setup(is_i);
    uint8_t* sb = ring + is_slot * C::kStageBytes;
    is_slot = is_slot == kStages - 1 ? 0 : is_slot + 1;
    if (++is_kt == nk) { is_kt = 0; ++is_i; }
    // the K tail: chunks at or past K copy zeros (K is a multiple of 8)
    const bool tail = k_tail && kt == nk - 1;
    const int kend = K - kt * kBK;   // valid elements of this stage's 64
#pragma unroll
    for (int gi = 0; gi < C::kWGroups; ++gi) {
      const uint16_t* src = wsrc[gi];
      if (tail && (lpos ^ swz((cw + C::kCopyWaves * gi) * 8 + lrow)) * 8 >= kend) src = zero;
      load_lds16(src, sb + (cw + C::kCopyWaves * gi) * 8 * kRowBytes);
      wsrc[gi] += wstep[gi];
    }
#pragma unroll
    for (int gi = 0; gi < C::kXGroups; ++gi) {
      const uint16_t* src = xsrc[gi];
      if (tail && (lpos ^ swz((cw + C::kCopyWaves * gi) * 8 + lrow)) * 8 >= kend) src = zero;
      load_lds16(src, sb + (kBN + (cw + C::kCopyWaves * gi) * 8) * kRowBytes);
      xsrc[gi] += xstep[gi];
    }
#pragma unroll
    for (int h = 0; h < C::kScaleCopies; ++h) {
      load_lds4(ssrc[h], sb + C::kOperandBytes + (cw + C::kCopyWaves * h) * 256);
      ssrc[h] += sstep[h];
    }
  };

  // ---- this wave's MFMA tiles ----
  // A tiles (weight rows): GEMM 1 gate rows wf*32 + {0, 16} and the matching
  // up rows kHalf + wf*32 + {0, 16}; GEMM 2 rows wf*64 + {0, 16, 32, 48}.
  // B tiles (pairs): the block's pairs are four quarters of BM/4; wave
  // group wp owns quarters wp and wp + 2 (B tiles j < NT/2 and j >= NT/2),
  // and skips the MFMAs of a quarter that holds only pads (the tail of an
  // expert's last block).  The four waves of a group sit on the four SIMDs,
  // so a block with one quarter of pairs takes about a quarter of the time.
  // Every tile starts at a multiple of 16 rows, so a lane's swizzle depends
  // only on r16 and each tile's offset is a constant added to one base per
  // operand and k half.
  constexpr int QS = BM / 4, TQ = NT / 2;   // pairs and B tiles per quarter
  const int wf = wv % C::kWF, wp = (wv / C::kWF) % C::kWP;
  const int r16 = lane & 15, kg = lane >> 4;
  auto brow = [&](int j) { return (j < TQ ? wp : wp + 2) * QS + 16 * (j % TQ); };
  const int arow0 = kGemm1 ? wf * 32 : wf * 64;
  int abase[2], bbase[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int slot = ((s * 4 + kg) ^ swz(r16)) << 4;
    abase[s] = (arow0 + r16) * kRowBytes + slot;
    bbase[s] = (wp * QS + r16) * kRowBytes + slot;   // from the B operand's first row
  }
  auto aconst = [](int i) {
    return (kGemm1 ? (i >> 1) * kHalf + (i & 1) * 16 : 16 * i) * kRowBytes;
  };

  f32x4 acc[4][NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: metadata of tiles 0 to 2, then the first kStages-1 stages ----
  issue_meta(0);
  issue_meta(1);
  issue_meta(2);
  wait_vmem<0>();
  __syncthreads();

  bool act0 = true, act1 = true;   // this wave's quarters hold a pair
  // MX: one scaled MFMA per (A tile, B tile) per stage; the lane's operand
  // is chunks kg and 4 + kg of its row, its scale byte that of k block kg.
  auto compute_mx = [&](const uint8_t* sb) {
    const uint8_t* sc = sb + C::kOperandBytes;
    const uint8_t* sbB = sb + kBN * kRowBytes;
    i32x8 af[4];
    int sa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = cat_u32x4(*reinterpret_cast<const u32x4*>(sb + abase[0] + aconst(i)),
                        *reinterpret_cast<const u32x4*>(sb + abase[1] + aconst(i)));
      const int row = arow0 + (kGemm1 ? (i >> 1) * kHalf + (i & 1) * 16 : 16 * i) + r16;
      sa[i] = sc[row * 4 + kg];
    }
    // B tiles one at a time (the A tiles stay in registers)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (!(q == 0 ? act0 : act1)) continue;
#pragma unroll
      for (int j = 0; j < TQ; ++j) {
        const int off = (q * 2 * QS + 16 * j) * kRowBytes;
        const i32x8 bfr = cat_u32x4(*reinterpret_cast<const u32x4*>(sbB + bbase[0] + off),
                                    *reinterpret_cast<const u32x4*>(sbB + bbase[1] + off));
        const int sbv = sc[(kBN + wp * QS + q * 2 * QS + 16 * j + r16) * 4 + kg];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][q * TQ + j] = mfma_mx_16x16x128(af[i], bfr, acc[i][q * TQ + j], sa[i], sbv);
      }
    }
  };
  // One stage of MFMAs over this wave's active quarters, fully unrolled;
  // sb holds the A rows (weights) and sbB the B rows (pairs) of the stage.
  auto compute = [&](const uint8_t* sb, const uint8_t* sbB) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(sb + abase[s] + aconst(i));
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (!(q == 0 ? act0 : act1)) continue;
        // B tiles in groups of JB (copy-wave kernels: fewer live registers)
        constexpr int JB = (kPC && TQ > 2) ? TQ / 2 : TQ;
#pragma unroll
        for (int j0 = 0; j0 < TQ; j0 += JB) {
          u32x4 bfr[JB];
#pragma unroll
          for (int j = 0; j < JB; ++j)
            bfr[j] = *reinterpret_cast<const u32x4*>(sbB + bbase[s] +
                                                     (q * 2 * QS + 16 * (j0 + j)) * kRowBytes);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < JB; ++j)
              acc[i][q * TQ + j0 + j] = mfma_16x16x32(af[i], bfr[j], acc[i][q * TQ + j0 + j]);
        }
      }
    }
  };
  // Consumption of stage g by an MFMA wave (after the stage's barrier):
  // MFMAs, and the tile epilogue after the tile's last k step.
  int c_i = 0, c_kt = 0, c_buf = 0, c_slot = 0, c_g = 0;
  auto consume = [&]() {
    const int i_tile = c_i, kt = c_kt;
    const int buf = c_buf;
    if (kt == 0) {
      const bool v0 = lane < QS && s_pair[buf][wp * QS + lane] < P;
      const bool v1 = lane < QS && s_pair[buf][(wp + 2) * QS + lane] < P;
      act0 = __ballot(v0) != 0ull;
      act1 = __ballot(v1) != 0ull;
    }
    if constexpr (QB > 0) {
      // quantized ring: A (widened weights) in two slots, B in kQXD + 1
      const uint8_t* sa = ring + (c_g & 1) * kQASlot;
      const uint8_t* sbb = ring + 2 * kQASlot + (c_g % (kQXD + 1)) * kQBSlot;
      if (act0 || act1) compute(sa, sbb);
    } else {
      const uint8_t* sb = ring + c_slot * C::kStageBytes;
      if (act0 || act1) {
        if constexpr (kMX) compute_mx(sb); else compute(sb, sb + kBN * kRowBytes);
      }
    }
    ++c_g;
    c_slot = c_slot == kStages - 1 ? 0 : c_slot + 1;
    if (++c_kt == nk) { c_kt = 0; ++c_i; c_buf = c_buf == kMeta - 1 ? 0 : c_buf + 1; }
    if (kt != nk - 1) return;

    // ---- tile epilogue: lane holds features 4*kg + q of each A tile, pair r16 of each B tile ----
    const int jt = j0 + i_tile * nslots;
    const int nt = jt - (jt / ntn) * ntn;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (!(j < TQ ? act0 : act1)) continue;
      const int p = s_pair[buf][brow(j) + r16];
      // 16-byte stores through a lane-pair exchange (not at 256 copy-wave
      // pairs, whose 168 registers leave no room)
      constexpr bool kStore16 = !(kPC && BM == 256);
      if constexpr (kStore16 && kGemm1) {
        // GEMM 1: lanes kg and kg ^ 1 swap halves so that the even lane
        // holds act columns 4 kg .. 4 kg + 7 of gate tile 0 and the odd lane
        // columns 4 (kg - 1) .. 4 kg + 3 of gate tile 1 (I % 8 == 0).
        const int I = prm.I;
        const bool odd = (kg & 1) != 0;
        u32x2 v[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const f32x4 gt = acc[i][j], up = acc[i + 2][j];
          v[i][0] = pack_bf16x2(silu_mul(gt[0], up[0]), silu_mul(gt[1], up[1]));
          v[i][1] = pack_bf16x2(silu_mul(gt[2], up[2]), silu_mul(gt[3], up[3]));
        }
        const u32x2 send = odd ? v[0] : v[1];
        u32x2 recv;
        recv[0] = __shfl_xor(send[0], 16, kWave);
        recv[1] = __shfl_xor(send[1], 16, kWave);
        const u32x4 o = odd ? u32x4{recv[0], recv[1], v[1][0], v[1][1]}
                            : u32x4{v[0][0], v[0][1], recv[0], recv[1]};
        const int n = nt * kHalf + wf * 32 + 16 * (odd ? 1 : 0) + 4 * (kg & ~1);
        if (p < P && n < I) *reinterpret_cast<u32x4*>(prm.out + (size_t)p * I + n) = o;
      } else if constexpr (kStore16) {
        // GEMM 2: 16-byte stores.  Lanes kg and kg ^ 1 (same pair) swap
        // halves so that, for A tiles i and i + 1, the even lane holds
        // features 4 kg .. 4 kg + 7 of tile i and the odd lane features
        // 4 (kg - 1) .. 4 kg + 3 of tile i + 1.
        const int H = prm.H;
        const bool odd = (kg & 1) != 0;
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          u32x2 v0, v1;
          v0[0] = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
          v0[1] = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
          v1[0] = pack_bf16x2(acc[i + 1][j][0], acc[i + 1][j][1]);
          v1[1] = pack_bf16x2(acc[i + 1][j][2], acc[i + 1][j][3]);
          const u32x2 send = odd ? v0 : v1;
          u32x2 recv;
          recv[0] = __shfl_xor(send[0], 16, kWave);
          recv[1] = __shfl_xor(send[1], 16, kWave);
          const u32x4 o = odd ? u32x4{recv[0], recv[1], v1[0], v1[1]}
                              : u32x4{v0[0], v0[1], recv[0], recv[1]};
          // H % 8 == 0 and h % 8 == 0: the 8 features exist or none do
          const int h = nt * kBN + wf * 64 + 16 * (i + (odd ? 1 : 0)) + 4 * (kg & ~1);
          if (p < P && h < H) *reinterpret_cast<u32x4*>(prm.out + (size_t)p * H + h) = o;
        }
      } else if (p < P) {
        if (kGemm1) {
          const int I = prm.I;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int n = nt * kHalf + wf * 32 + 16 * i + 4 * kg;
            if (n >= I) continue;
            const f32x4 gt = acc[i][j], up = acc[i + 2][j];
            u32x2 v;
            v[0] = pack_bf16x2(silu_mul(gt[0], up[0]), silu_mul(gt[1], up[1]));
            v[1] = pack_bf16x2(silu_mul(gt[2], up[2]), silu_mul(gt[3], up[3]));
            *reinterpret_cast<u32x2*>(prm.out + (size_t)p * I + n) = v;
          }
        } else {
          const int H = prm.H;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int h = nt * kBN + wf * 64 + 16 * i + 4 * kg;
            if (h >= H) continue;
            u32x2 v;
            v[0] = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
            v[1] = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
            *reinterpret_cast<u32x2*>(prm.out + (size_t)p * H + h) = v;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // ---- quantized weights (QB > 0): copy waves and widen waves ----
  // Copy waves DMA stage h's codes (and, at the start of a scale block, one
  // aligned 32-bit word of the scales and one of the biases per weight row)
  // three stages ahead, and its gathered pair rows kQXD stages ahead, and
  // wait for them to land before the barriers: the codes of stage h by
  // barrier h - 1, the pair rows by barrier h.  Between barriers h - 1 and h
  // each lane of the widen waves widens one weight row of stage h, w = s q + b
  // rounded to bf16, into the stage's A slot in the layout the copies of bf16
  // weights give (chunk c of row R at slot c ^ swz(R)), while the MFMA waves
  // multiply stage h - 1.  Separate waves, so copies that stall at issue
  // never delay the widening.  A scale block is two stages when the group
  // count per row is even (every row's word then starts at an even group),
  // else one stage, with the half picked per row.  Codes use the default
  // cache policy: a 128-byte line of codes serves 128 / kQCB stages.
  [[maybe_unused]] constexpr int kQI = kQCSlot / 1024 / C::kCopyWaves;   // code copies per wave and stage
  [[maybe_unused]] constexpr int kQRows = 1024 / kQCB;                  // code rows per copy
  [[maybe_unused]] constexpr int kQChunks = kQCB / 16;                  // 16-byte chunks per code row and stage
  uint8_t* const qa = ring;                                             // 2 A slots
  uint8_t* const qb = ring + 2 * kQASlot;                               // kQXD + 1 B slots
  uint8_t* const qc = qb + (kQXD + 1) * kQBSlot;                        // 3 code slots
  uint8_t* const qs = qc + 3 * kQCSlot;                                 // 3 scale slots
  const int ng = Ke / 64;
  const int sb = (ng & 1) == 0 ? 2 : 1;                                 // stages per scale block
  const int R = cw * 64 + lane;            // the weight row whose codes and words this lane moves
  // global weight row of tile row r of tile i (or -1 past the weights)
  auto wrow = [&](int i, int r) -> long long {
    const int j = j0 + i * nslots;
    const int nt = j - (j / ntn) * ntn;
    const int e = s_exp[i % kMeta];
    if (kGemm1) {
      const int f = nt * kHalf + (r % kHalf);
      return f < prm.I ? (long long)e * 2 * prm.I + (r < kHalf ? f : prm.I + f) : -1;
    }
    const int h = nt * kBN + r;
    return h < prm.H ? (long long)e * prm.H + h : -1;
  };

  auto quant_copier = [&]() {
    if constexpr (QB > 0) {
      constexpr int kX = C::kXGroups;                      // pair-row copies per wave and stage
      const int rowq = Ke * QB / 8;                        // code bytes per weight row
      const uint8_t* csrc[kQI];
      long long srow = -1;                                 // this lane's scale row (R)
      int q_i = 0, q_kt = 0, q_h = 0, nsb = 0, x_h = 0, x_i = 0, x_kt = 0;
      // Codes (and the scale block's words) of the next stage; returns the
      // number of memory operations (0 past the last stage).
      auto issue_codes = [&]() -> int {
        if (q_h >= G) return 0;
        if (q_kt == 0) {
          issue_meta(q_i + 3);
#pragma unroll
          for (int q = 0; q < kQI; ++q) {
            const int r = (cw * kQI + q) * kQRows + lane / kQChunks;
            const long long wr = wrow(q_i, r);
            csrc[q] = wr >= 0 ? prm.wq + wr * rowq + (lane % kQChunks) * 16 : nullptr;
          }
          srow = wrow(q_i, R);
        }
        const int kt = q_kt, h = q_h++;
        if (++q_kt == nk) { q_kt = 0; ++q_i; }
        uint8_t* cdst = qc + (h % 3) * kQCSlot;
#pragma unroll
        for (int q = 0; q < kQI; ++q)
          load_lds16(csrc[q] != nullptr ? (const void*)(csrc[q] + kt * kQCB)
                                        : (const void*)kZeroPage,
                     cdst + (cw * kQI + q) * 1024);
        if (kt % sb != 0) return kQI;
        // the aligned word holding group kt of row R (sb = 2: groups kt, kt + 1)
        const long long el = srow >= 0 ? srow * ng + kt : 0;
        uint8_t* sdst = qs + (nsb++ % 3) * kQSSlot;
        load_lds4(srow >= 0 ? (const void*)(prm.wsc + (el & ~1ll) * 2) : (const void*)kZeroPage,
                  sdst + cw * 256);
        load_lds4(srow >= 0 ? (const void*)(prm.wbi + (el & ~1ll) * 2) : (const void*)kZeroPage,
                  sdst + 1024 + cw * 256);
        return kQI + 2;
      };
      // Pair rows of the next stage; returns the operation count.
      auto issue_rows = [&]() -> int {
        if (x_h >= G) return 0;
        if (x_kt == 0) setup_x(x_i);
        if (++x_kt == nk) { x_kt = 0; ++x_i; }
        uint8_t* bdst = qb + (x_h++ % (kQXD + 1)) * kQBSlot;
#pragma unroll
        for (int gi = 0; gi < kX; ++gi) {
          load_lds16(xsrc[gi], bdst + (cw + C::kCopyWaves * gi) * 8 * kRowBytes);
          xsrc[gi] += xstep[gi];
        }
        return kX;
      };
      // at most n memory operations of this wave pending; n is one of the
      // sizes a run of the latest copies can have (else: wait for all)
      auto wait_n = [&](int n) {
        if (n == 0) wait_vmem<0>();
        else if (n == kX) wait_vmem<kX>();
        else if (n == kQI) wait_vmem<kQI>();
        else if (n == kQI + 2) wait_vmem<kQI + 2>();
        else if (n == kX + kQI) wait_vmem<kX + kQI>();
        else if (n == kX + kQI + 2) wait_vmem<kX + kQI + 2>();
        else if (n == 2 * kX + 2 * kQI) wait_vmem<2 * kX + 2 * kQI>();
        else if (n == 2 * kX + 2 * kQI + 2) wait_vmem<2 * kX + 2 * kQI + 2>();
        else if (n == 2 * kX + 2 * kQI + 4) wait_vmem<2 * kX + 2 * kQI + 4>();
        else wait_vmem<0>();
      };
      // Batch b = rows(b + kQXD), codes(b + 3); batches -2 and -1 after
      // codes(0) before the first barrier, batch b >= 0 after barrier b.
      // Before barrier b + 1, codes(b + 2) (batch b - 1) and rows(b + 1)
      // (batch b + 1 - kQXD) must have landed: all but the last batch's
      // operations (kQXD = 2), or all but its codes' (kQXD = 1).
      issue_codes();
      const int r2 = kQXD == 2 ? issue_rows() : 0;   // batch -2
      const int c2 = issue_codes();
      int r1 = issue_rows();                         // batch -1
      int c1 = issue_codes();
      wait_n(r2 + c2 + r1 + c1);                     // codes(0)
      barrier_nofence();                             // barrier -1
      wait_n((kQXD == 2 ? r1 : 0) + c1);             // codes(1), rows(0)
      wait_lgkm0();
      barrier_nofence();                             // barrier 0
      for (int g = 0; g + 1 < G; ++g) {
        r1 = issue_rows();                           // batch g
        c1 = issue_codes();
        wait_n((kQXD == 2 ? r1 : 0) + c1);           // codes(g + 2), rows(g + 1)
        barrier_nofence();                           // barrier g + 1
      }
      wait_vmem<0>();                                // no copy outlives the wave
    }
  };

  auto quant_widener = [&]() {
    if constexpr (QB > 0) {
      int w_i = 0, w_kt = 0, wsb = -1;
      long long wr = -1;                                   // global row of R in the current tile
      barrier_nofence();                                   // barrier -1: codes(0) are in LDS
      for (int g = 0; g < G; ++g) {
        const int kt = w_kt;
        if (kt == 0) wr = wrow(w_i, R);
        if (++w_kt == nk) { w_kt = 0; ++w_i; }
        if (kt % sb == 0) ++wsb;
        const uint8_t* cr = qc + (g % 3) * kQCSlot + R * kQCB;
        const uint8_t* ss = qs + (wsb % 3) * kQSSlot;
        const uint32_t swd = *reinterpret_cast<const uint32_t*>(ss + R * 4);
        const uint32_t bwd = *reinterpret_cast<const uint32_t*>(ss + 1024 + R * 4);
        // the half of the word holding group kt (rows past the weights read 0)
        const int half = sb == 2 ? (kt & 1) : (int)((wr >= 0 ? wr * ng + kt : 0) & 1);
        const float sc = half ? bf16_hi(swd) : bf16_lo(swd);
        const float bi = half ? bf16_hi(bwd) : bf16_lo(bwd);
        uint8_t* arow = qa + (g & 1) * kQASlot + R * kRowBytes;
        u32x4 cw4[kQCB / 16];
#pragma unroll
        for (int i = 0; i < kQCB / 16; ++i) cw4[i] = *reinterpret_cast<const u32x4*>(cr + 16 * i);
#pragma unroll
        for (int c = 0; c < 8; ++c) {      // 8 values a chunk, 8 chunks of 64 k
          float v[8];
          if constexpr (QB == 4) {
            // nibble 2j is byte j of lo, nibble 2j + 1 byte j of hi; the
            // empty asm hides that their bytes are below 16, so the byte
            // conversions (one instruction each) stay
            uint32_t lo = cw4[c >> 2][c & 3] & 0x0F0F0F0Fu;
            uint32_t hi = (cw4[c >> 2][c & 3] >> 4) & 0x0F0F0F0Fu;
            asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              v[2 * k] = (float)((lo >> (8 * k)) & 255u);
              v[2 * k + 1] = (float)((hi >> (8 * k)) & 255u);
            }
          } else {
            const uint32_t w0 = cw4[c >> 1][(c & 1) * 2], w1 = cw4[c >> 1][(c & 1) * 2 + 1];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              v[k] = (float)((w0 >> (8 * k)) & 255u);
              v[4 + k] = (float)((w1 >> (8 * k)) & 255u);
            }
          }
          u32x4 o;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            o[k] = pack_bf16x2(__builtin_fmaf(sc, v[2 * k], bi), __builtin_fmaf(sc, v[2 * k + 1], bi));
          *reinterpret_cast<u32x4*>(arow + ((c ^ swz(R)) << 4)) = o;
        }
        wait_lgkm0();        // this lane's A rows of stage g are in LDS
        barrier_nofence();   // barrier g
      }
    }
  };

  if constexpr (kPC) {
    // Copy waves and MFMA waves run separate loops with the same barriers,
    // so neither keeps the other's registers live.
    if (copier && QB > 0) {
      quant_copier();
    } else if (widener) {
      quant_widener();
    } else if (copier) {
#pragma unroll
      for (int g = 0; g < kStages - 1; ++g)
        if (g < G) issue_stage();
      for (int g = 0; g < G; ++g) {
        // stage g has landed once at most the later stages' copies are pending
        if (kStages == 3 && g + 1 < G) wait_vmem<C::kLoads>(); else wait_vmem<0>();
        barrier_nofence();   // stage g is in LDS; stage g-1 has been consumed
        if (g + kStages - 1 < G) issue_stage();
      }
    } else {
      if (QB > 0) barrier_nofence();   // barrier -1 (the widen waves start stage 0)
      // bf16 GEMM 1: the MFMA waves take issue priority over the copy wave
      // of their SIMD (measured: GEMM 1 2-4 % faster; GEMM 2, the MXFP8 and
      // the quantized tiles gain nothing)
      if constexpr (kGemm1 && QB == 0 && !kMX) __builtin_amdgcn_s_setprio(1);
      for (int g = 0; g < G; ++g) {
        barrier_nofence();
        consume();
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < kStages - 1; ++g)
      if (g < G) issue_stage();
    for (int g = 0; g < G; ++g) {
      // stage g has landed once at most the later stages' copies are pending
      if (kStages == 3 && g + 1 < G) wait_vmem<C::kLoads>(); else wait_vmem<0>();
      // Every wave's part of stage g is in LDS, and stage g-1 is consumed.
      barrier_nofence();
      if (g + kStages - 1 < G) issue_stage();
      consume();
    }
  }
}

// out[t, h] = bf16(sum over slots j of topk_weights[t, j] * rows[t*top_k + j, h]),
// j ascending, fp32 sum.  Page "Mixture of Experts in vLLM ...", section
// "Put the results back, and combine them per token".  Thread: 8
// consecutive columns of one token (H % 8 == 0).
__global__ __launch_bounds__(256) void combine_rows_kernel(const uint16_t* __restrict__ rows,
                                                           const float* __restrict__ topk_weights,
                                                           int M, int top_k, int H,
                                                           uint16_t* __restrict__ out) {
  const int h8 = H / 8;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)M * h8) return;
  const int t = (int)(i / h8), h = (int)(i - (long long)t * h8) * 8;
  const uint16_t* src = rows + (size_t)t * top_k * H + h;
  // all top_k row loads leave before the first add
  constexpr int kMaxK = 32;
  u32x4 part[kMaxK];
  float wt[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < top_k) {
      part[j] = *reinterpret_cast<const u32x4*>(src + (size_t)j * H);
      wt[j] = topk_weights[(size_t)t * top_k + j];
    }
  float sum[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) sum[q] = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < top_k) {
      const float w = wt[j];
      const u32x4 v = part[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sum[2 * q] += w * __uint_as_float(v[q] << 16);
        sum[2 * q + 1] += w * __uint_as_float(v[q] & 0xffff0000u);
      }
    }
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(sum[2 * q], sum[2 * q + 1]);
  *reinterpret_cast<u32x4*>(out + (size_t)t * H + h) = o;
}

template <int BM, bool kGemm1, bool kMX = false, bool kPC = false, int QB = 0>
hipError_t launch_tiled(const moe_host::GemmArgs& a, hipStream_t s, uint16_t* out,
                        const moe_host::QGemmArgs* q = nullptr) {
  using C = TileCfg<BM, kMX, kPC>;
  constexpr int kBN = C::kBN;
  TileParams prm{};
  prm.a_src = a.a_src;
  prm.w = a.w;
  prm.a_scales = a.a_scales;
  prm.w_scales = a.w_scales;
  prm.sorted = a.sorted_token_ids;
  prm.expert_ids = a.expert_ids;
  prm.boff = a.expert_block_offsets;
  prm.M = a.M;
  prm.top_k = a.top_k;
  prm.E = a.E;
  prm.H = a.H;
  prm.I = a.I;
  prm.ntn = kGemm1 ? moe_host::ceil_div_host(a.I, kBN / 2) : moe_host::ceil_div_host(a.H, kBN);
  prm.out = out;
  if (QB > 0) {
    prm.wq = reinterpret_cast<const uint8_t*>(kGemm1 ? q->w13q : q->w2q);
    prm.wsc = reinterpret_cast<const uint8_t*>(kGemm1 ? q->w13_scales : q->w2_scales);
    prm.wbi = reinterpret_cast<const uint8_t*>(kGemm1 ? q->w13_biases : q->w2_biases);
    prm.w = reinterpret_cast<const uint16_t*>(prm.wq);   // (no bf16 weights are read)
  }
  // persistent grid: one workgroup per CU, never more than the tiles, a multiple of 8
  const long long tiles = (long long)a.max_blocks * prm.ntn;
  long long grid = std::min<long long>(tiles, moe_host::device_cu_count());
  grid = std::max<long long>(8, (grid + 7) / 8 * 8);
  // quantized ring: 2 A slots, 3 (8 bits: 2) B slots, 3 code slots, 3 scale slots
  const size_t lds = QB > 0 ? (size_t)2 * kBN * kRowBytes + (QB == 8 ? 2 : 3) * BM * kRowBytes +
                                  3 * kBN * (kBK * QB / 8) + 3 * kBN * 8
                            : C::kRingBytes;
  static bool lds_set[moe_host::kMaxDevices] = {};
  const hipError_t err = moe_host::ensure_dynamic_lds(
      reinterpret_cast<const void*>(&gemm_tiled_kernel<BM, kGemm1, kMX, kPC, QB>), (int)lds, lds_set);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((gemm_tiled_kernel<BM, kGemm1, kMX, kPC, QB>), dim3((unsigned)grid),
                     dim3(QB > 0 ? 1024 : C::kThreadsT), lds, s, prm);
  return hipGetLastError();
}

}  // namespace

namespace moe_host {

hipError_t launch_gemm1_tiled(const GemmArgs& a, hipStream_t s) {
  if (a.mx) {
    if (a.block_m == 256) return launch_tiled<256, true, true>(a, s, a.out);
    if (a.block_m == 128) return launch_tiled<128, true, true, true>(a, s, a.out);
    return launch_tiled<64, true, true>(a, s, a.out);
  }
  if (a.block_m == 256) return launch_tiled<256, true, false, true>(a, s, a.out);
  if (a.block_m == 128) return launch_tiled<128, true, false, true>(a, s, a.out);
  return launch_tiled<64, true, false, true>(a, s, a.out);
}

namespace {
GemmArgs quant_gemm_args(const QGemmArgs& q) {
  GemmArgs a{};
  a.sorted_token_ids = q.sorted_token_ids;
  a.expert_ids = q.expert_ids;
  a.expert_block_offsets = q.expert_block_offsets;
  a.topk_weights = q.topk_weights;
  a.M = q.M;
  a.top_k = q.top_k;
  a.E = q.E;
  a.H = q.H;
  a.I = q.I;
  a.block_m = 128;
  a.max_blocks = q.max_blocks;
  return a;
}
}  // namespace

hipError_t launch_qgemm1_tiled(const QGemmArgs& q, hipStream_t s) {
  GemmArgs a = quant_gemm_args(q);
  a.a_src = q.x;
  return q.bits == 4 ? launch_tiled<128, true, false, true, 4>(a, s, q.act, &q)
                     : launch_tiled<128, true, false, true, 8>(a, s, q.act, &q);
}

hipError_t launch_qgemm2_tiled(const QGemmArgs& q, hipStream_t s) {
  GemmArgs a = quant_gemm_args(q);
  a.a_src = q.act;
  uint16_t* rows = reinterpret_cast<uint16_t*>(q.partial);
  const hipError_t err = q.bits == 4 ? launch_tiled<128, false, false, true, 4>(a, s, rows, &q)
                                     : launch_tiled<128, false, false, true, 8>(a, s, rows, &q);
  if (err != hipSuccess) return err;
  const long long n8 = (long long)q.M * (q.H / 8);
  hipLaunchKernelGGL(combine_rows_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, rows,
                     q.topk_weights, q.M, q.top_k, q.H, q.out);
  return hipGetLastError();
}

hipError_t launch_gemm2_tiled(const GemmArgs& a, hipStream_t s) {
  uint16_t* rows = reinterpret_cast<uint16_t*>(a.partial);
  hipError_t err;
  if (a.mx)
    err = a.block_m == 256   ? launch_tiled<256, false, true>(a, s, rows)
          : a.block_m == 128 ? launch_tiled<128, false, true, true>(a, s, rows)
                             : launch_tiled<64, false, true>(a, s, rows);
  else
    err = a.block_m == 256   ? launch_tiled<256, false, false, true>(a, s, rows)
          : a.block_m == 128 ? launch_tiled<128, false, false, true>(a, s, rows)
                             : launch_tiled<64, false, false, true>(a, s, rows);
  if (err != hipSuccess) return err;
  const long long n8 = (long long)a.M * (a.H / 8);
  hipLaunchKernelGGL(combine_rows_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, rows,
                     a.topk_weights, a.M, a.top_k, a.H, a.out);
  return hipGetLastError();
}

}  // namespace moe_host
