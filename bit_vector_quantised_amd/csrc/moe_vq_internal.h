// Internal definitions shared by the MoE-VQ HIP kernels and the C-ABI host code.
// Target: AMD Instinct MI355X (gfx950, CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_vq.h"

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef short bf16x2_t __attribute__((ext_vector_type(2)));

namespace mvq {

// Activations are staged for the decode products as fp16 with one power-of-two
// factor per token and per SLICE consecutive columns (exact for bf16 inputs).
constexpr int SLICE = 1024;
constexpr int MAX_E = 1024;
constexpr int MAX_K = 32;
constexpr int MAX_T = 65536;
constexpr int MAX_DIM = 16384;

// Signed codebook table in LDS: 256 entries (word b -> sgn(b) * CB[b & 0x7F]) of four
// fp16 values, replicated TAB_COPIES times so that lane l reads copy (l & 31) and
// every lane of a half-wave hits its own pair of banks:
//     byte address(b, lane) = b * 256 + (lane & 31) * 8
// The address is one v_perm_b32: the word's byte goes to bits 8..15, the lane
// offset (< 256) stays in bits 0..7.
constexpr int TAB_COPIES = 32;
constexpr int TAB_BYTES = 256 * TAB_COPIES * 8;  // 64 KiB

// Workspace header words.
enum HdrField {
  HDR_STATUS = 0,     // first device error (moe_vq_status), 0 = OK
  HDR_INFO = 1,       // offending expert id or -1
  HDR_N_ACTIVE = 2,   // number of distinct selected experts
  HDR_N_PAIRS = 3,    // routed (token, expert) pairs placed in the worklist
  HDR_N_TOKENS = 4,
  HDR_GROUPS1 = 5,    // FC1 token groups (sum over active experts of ceil(m / MT1))
  HDR_GROUPS2 = 6,    // FC2 token groups
  HDR_MT1 = 7,
  HDR_MT2 = 8,
  HDR_KEY = 9,        // shape key of the step that built the worklist
  HDR_X_LO = 10,      // address of the activations the step was routed with (low, high
  HDR_X_HI = 11,      // word) and their dtype: FC1 and prefill read the staged copy of x
  HDR_X_DTYPE = 12,   // and refuse a call made with other activations
  HDR_PGRID1 = 13,    // grid the FC1 tile split was made for (0: no split)
  HDR_PGRID2 = 14,    // the same for FC2
  HDR_WORDS = 64
};

// Shape key written by the worklist and checked by the FC kernels, so that a workspace
// that was never routed (or was routed for other shapes) is rejected instead of read.
__host__ __device__ inline uint32_t shape_key(int T, int E, int k, int H, int I) {
  uint32_t h = 2166136261u;
  const int v[5] = {T, E, k, H, I};
  for (int i = 0; i < 5; ++i) { h ^= (uint32_t)v[i]; h *= 16777619u; }
  return h | 1u;
}

__host__ __device__ inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Byte offsets of the six blocks of one expert slot (relative to the slot start).
struct SlotLayout {
  uint64_t q_gate, q_up, q_down, s_gate, s_up, s_down, total;
};

__host__ __device__ inline SlotLayout slot_layout(int fmt, int H, int I) {
  SlotLayout L{};
  uint64_t qg, qd, sg, sd;
  if (fmt == MOE_VQ_FMT_VQ2) {
    qg = (uint64_t)I * (H / 4); qd = (uint64_t)H * (I / 4);
    sg = (uint64_t)I * (H / 128) * 2; sd = (uint64_t)H * (I / 128) * 2;
  } else {  // MXFP4
    qg = (uint64_t)I * (H / 2); qd = (uint64_t)H * (I / 2);
    sg = (uint64_t)I * (H / 32); sd = (uint64_t)H * (I / 32);
  }
  uint64_t off = 0;
  L.q_gate = off; off = align256(off + qg);
  L.q_up = off;   off = align256(off + qg);
  L.q_down = off; off = align256(off + qd);
  L.s_gate = off; off = align256(off + sg);
  L.s_up = off;   off = align256(off + sg);
  L.s_down = off; off = align256(off + sd);
  L.total = off;
  return L;
}

__host__ __device__ inline int n_slices(int n) { return (n + SLICE - 1) / SLICE; }

constexpr int MAX_MT = 4;  // largest token group of the vector-ALU FC kernels
constexpr int MF_MT = 16;  // token group of the matrix-core FC kernel (its A operand rows)

// K of the matrix-core FC kernel it is built for (FC2 holds its fp32 activations for a
// whole quarter of K in registers, which caps K at 2048 there).
__host__ __device__ inline bool mf_supported(int K, bool fc1) {
  return K == 1024 || K == 2048 || (fc1 && K == 7168);
}

// Rows of one tile of the matrix-core FC kernel at K = 1024 cpl: 16-row blocks, as many
// as keep several KB of codes in flight per wave within the registers of eight waves
// (FC1 at most 4, FC2 at most 8; at K = 7168 FC1 takes one block).
__host__ __device__ constexpr int mf_tile_rows(int cpl, bool fc1) {
  const int rule = cpl >= 4 ? (fc1 ? 1 : 2) : (fc1 ? 8 / cpl : 16 / cpl);
  const int cap = fc1 ? 4 : 8;
  return 16 * (rule < cap ? rule : cap);
}

// Workgroups of a matrix-core FC launch: one per compute unit, at most one per tile.
__host__ __device__ inline int mf_grid(int n_cu, int max_groups, int nrows, int rows) {
  const long tiles = (long)max_groups * ((nrows + rows - 1) / rows);
  return (int)(tiles < n_cu ? tiles : n_cu);
}

// The worklist splits the matrix-core FC kernels' tiles over their workgroups by cost
// rather than by count (table of MAX_PART + 1 tile boundaries per kernel): a tile of an
// MXFP4 group reads twice the bytes of a VQ2 one and, starting with nothing in flight,
// takes longer still, so equal tile counts left the workgroups holding MXFP4 tiles
// running about twice as long as the rest.  The cost ratio 5 : 2 was the fastest of 1.5
// to 4 for both a mixed-format batch and FP4 delta-cache copies.
constexpr int MAX_PART = 1024;
constexpr int PART_COST_VQ2 = 2, PART_COST_MX4 = 5, PART_COST_ABSENT = 1;
__host__ __device__ inline int part_cost(uint32_t fmt) {
  return fmt == MOE_VQ_FMT_VQ2 ? PART_COST_VQ2 : (fmt == MOE_VQ_FMT_MXFP4 ? PART_COST_MX4 : PART_COST_ABSENT);
}

// One token group of one expert, as the FC kernels consume it: a tile is (group, block
// of rows), so a tile reads one record to know where its codes and tokens are.
struct __align__(16) GroupRec {
  uint64_t slot_off;      // byte offset of the expert's slot in the pool
  int32_t p0;             // first entry of the group in pair_list
  int32_t mcount;         // tokens in the group (1..MT)
  uint32_t fmt;           // slot format (MOE_VQ_FMT_ABSENT when not resident)
  int32_t expert;
  int32_t pair[MAX_MT];   // its first pair indices p = t*k + i (repeats the last when short)
  int32_t pad[4];
};

// FC decode-path geometry shared by host and kernels.
constexpr int FC_THREADS = 256;
constexpr int LDS_LIMIT = 160 * 1024;

// Staged activations in LDS: each 64-value fp16 chunk (128 B) is padded to 144 B so
// that the 16 lanes of a row, which read 16 consecutive chunks, hit 16 distinct groups
// of 4 banks.
constexpr int XCHUNK_UNITS = 9;  // 16-byte units per padded chunk
__host__ __device__ inline size_t fc_x_units(int K) { return (size_t)(K / 64) * XCHUNK_UNITS; }
__host__ __device__ inline int x_unit(int u) { return (u >> 3) * XCHUNK_UNITS + (u & 7); }

// LDS of one FC workgroup: table, padded activations, their slice factors and the
// per-wave reduction slots, rounded up to the 512-byte allocation granularity.
__host__ __device__ inline size_t fc_lds_bytes(int MT, int K) {
  const size_t b = (size_t)TAB_BYTES + (size_t)MT * fc_x_units(K) * 16 + (size_t)MT * n_slices(K) * 4 +
                   (size_t)4 * MT * n_slices(K) * 4;
  return (b + 511) & ~(size_t)511;
}

// Tokens of one expert that share one pass over its codes: one token alone (the
// vector-ALU stream kernel), else up to 16 on the matrix-core kernel where it is built
// for K, else up to 4 on the vector-ALU kernels.
__host__ __device__ inline int fc_group_tokens(int n_tokens, int K, bool fc1) {
  if (n_tokens > 1 && mf_supported(K, fc1)) return MF_MT;
  int mt = n_tokens <= 1 ? 1 : 4;
  while (mt > 1 && fc_lds_bytes(mt, K) > (size_t)LDS_LIMIT) mt >>= 1;
  return mt;
}

// Upper bound on the token groups the worklist can produce.
__host__ __device__ inline int fc_max_groups(int T, int k, int E, int MT) {
  const long P = (long)T * k;
  const long act = P < E ? P : E;
  return (int)((P + act * (MT - 1)) / MT);
}

// Prefill (grouped matrix-core GEMM) geometry.
constexpr int PF_BM = 64;    // tokens of one expert per tile
constexpr int PF_KG = 128;   // reduction step: one scale group

__host__ __device__ inline int pf_rows_per_tile(bool fc1) { return fc1 ? 128 : 256; }

// Upper bound on the prefill token tiles: each active expert adds at most one partial tile.
__host__ __device__ inline int pf_max_mtiles(int T, int k, int E) {
  const long P = (long)T * k;
  const long act = P < E ? P : E;
  return (int)(P / PF_BM + act);
}

// Workspace layout for (E, H, I, k, T).  EV: the experts the worklist can list (E, or 2E
// with an FP4 delta cache, whose copies are listed as experts E + e).
struct WsLayout {
  size_t hdr, logits, x_h, x_sc, act_expert, act_start, act_off, act_fmt, grp1, grp2, rec1, rec2,
      part1, part2, pair_list, pair_w, o_buf, x16, x16_e, mt_pre, hmax, h_pre, total;
  int KS;  // number of activation slices of H
  int MT1, MT2, G1, G2;
};

inline WsLayout ws_layout(int E, int H, int I, int k, int T, int EV = 0) {
  WsLayout L{};
  if (EV < E) EV = E;
  size_t P = (size_t)T * k;
  L.KS = n_slices(H);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  L.hdr = take(HDR_WORDS * 4);
  // the distinct experts follow the header directly (HDR_WORDS * 4 is 256 bytes), so the
  // host reads both back in one copy
  L.act_expert = take((size_t)EV * 4);
  L.logits = take((size_t)((L.KS + 3) & ~3) * T * E * 4);  // [T][E][KS rounded to 4]
  L.x_h = take((size_t)T * H * 2);
  L.x_sc = take((size_t)T * L.KS * 4);
  L.act_start = take((size_t)(EV + 1) * 4);
  L.act_off = take((size_t)EV * 8);
  L.act_fmt = take((size_t)EV * 4);
  L.grp1 = take((size_t)(EV + 1) * 4);
  L.grp2 = take((size_t)(EV + 1) * 4);
  L.MT1 = fc_group_tokens(T, H, true);
  L.MT2 = fc_group_tokens(T, I, false);
  L.G1 = fc_max_groups(T, k, EV, L.MT1);
  L.G2 = fc_max_groups(T, k, EV, L.MT2);
  L.rec1 = take((size_t)L.G1 * sizeof(GroupRec));
  L.rec2 = take((size_t)L.G2 * sizeof(GroupRec));
  L.part1 = take((size_t)(MAX_PART + 1) * 4);
  L.part2 = take((size_t)(MAX_PART + 1) * 4);
  L.pair_list = take(P * 4);
  L.pair_w = take(P * 4);
  L.o_buf = take(P * H * 4);
  // prefill: activations as fp16 with one power-of-two factor per token, the token-tile
  // prefix over the active experts, the per-pair max |h| and h itself
  L.x16 = take((size_t)T * H * 2);
  L.x16_e = take((size_t)T * 4);
  L.mt_pre = take((size_t)(EV + 1) * 4);
  L.hmax = take(P * 4);
  L.h_pre = take(P * I * 2);
  L.total = off;
  return L;
}

// Kernel argument bundles -------------------------------------------------------------

struct RouteArgs {
  const uint16_t* router_w;  // bf16 [E][H]
  const void* x;             // [T][H] f32 or bf16
  int T, H, E, k, KS;
  int ksp;                   // partial sums per (token, expert): KS rounded up to 4, or 1
  float* logits;             // [T][E][ksp] partial sums
  uint16_t* x_h;             // [T][H] fp16 bits
  float* x_sc;               // [T][KS]
  int32_t* topk_ids;         // [T][k]
  float* topk_w;             // [T][k]
  float* pair_w;             // [T][k]
};

struct WorklistArgs {
  const void* x;             // the activations routed (recorded in the header)
  int x_dtype;
  const int32_t* topk_ids;
  const moe_vq_slot* slots;
  const moe_vq_slot* delta_slots;  // FP4 copies, or null (no delta cache)
  const float* pair_w;             // [T*k] routing weights (the gate reads them)
  float tau;                       // confidence gate of the delta cache
  uint64_t pool_bytes;
  int T, E, k, H, I, MT1, MT2;
  int EV;                          // experts the worklist can list: E, or 2E with copies
  int32_t* part1;                  // FC1 / FC2 tile split by cost (MAX_PART + 1 entries)
  int32_t* part2;
  int grid1, grid2;                // the matrix-core launches' grids (0: no split)
  int rb1, rb2;                    // their row blocks per token group
  uint32_t* hdr;
  int32_t* act_expert;
  int32_t* act_start;
  uint64_t* act_off;
  uint32_t* act_fmt;
  int32_t* grp1;
  int32_t* grp2;
  GroupRec* rec1;
  GroupRec* rec2;
  int G1, G2;
  int32_t* pair_list;
  uint32_t key;
};

struct FcArgs {
  const uint8_t* pool;
  const uint16_t* codebook;  // fp16 [128][4]
  uint32_t* hdr;             // read; the status word is written when the call is refused
  const int32_t* act_start;
  const uint64_t* act_off;
  const uint32_t* act_fmt;
  const int32_t* grp;        // group prefix for this kernel's MT
  const GroupRec* rec;       // group records for this kernel's MT
  const int32_t* pair_list;
  const float* pair_w;
  const uint16_t* x_h;       // FC1: staged activations [T][H] fp16
  const float* x_sc;         // FC1: [T][KS]
  const float* h_in;         // FC2: [P][I] fp32
  float* out;                // FC1: h [P][I]; FC2: o_buf [P][H]
  float* y;                  // FC2: [T][H]
  int T, H, I, k, KS, E;
  uint32_t key;
  int max_groups;            // upper bound on token groups for this T
  uint64_t x_addr;           // FC1: the activations the caller passes (must be the routed ones)
  int x_dtype;
  float lim;                 // FC1: SwiGLU clamp (0: none)
  int accumulate;            // FC2: add to y instead of overwriting it
  const int32_t* part;       // matrix-core kernel: the worklist's tile split, or null
  SlotLayout vq2, mx4;
};

struct PrefillArgs {
  const uint8_t* pool;
  const uint16_t* codebook;  // fp16 [128][4]
  uint32_t* hdr;             // read; the status word is written when the call is refused
  const int32_t* act_start;  // [n_active + 1] first pair of each active expert
  const uint64_t* act_off;
  const uint32_t* act_fmt;
  const int32_t* pair_list;
  const float* pair_w;
  const void* x;             // [T][H] f32 or bf16
  uint16_t* x16;             // [T][H] fp16 bits
  int32_t* x16_e;            // [T] x = x16 * 2^e
  int32_t* mt_pre;           // [E + 1] token-tile prefix over active experts
  uint32_t* hmax;            // [P] bits of max |h| per pair
  uint16_t* h;               // [P][I] bf16 (FC1 output, FC2 input)
  float* o_buf;              // [P][H]
  float* y;                  // [T][H]
  int T, H, I, k, E;
  int x_dtype;
  float lim;                 // SwiGLU clamp (0: none)
  uint32_t key;
  SlotLayout vq2, mx4;
};

// A workspace that was routed for this call: the shape key, and (FC1, prefill) the same
// activations.  Header words are read together, before any is tested.
__host__ __device__ inline bool x_matches(uint32_t lo, uint32_t hi, uint32_t dt, uint64_t addr, int dtype) {
  return (lo == (uint32_t)addr) & (hi == (uint32_t)(addr >> 32)) & (dt == (uint32_t)dtype);
}

}  // namespace mvq
