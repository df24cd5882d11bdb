// sv_internal.h — argument blocks and workspace records shared by the host
// launchers and the kernels of the verify library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kMaxVecsPerThread = 8;  // 16-byte vectors per thread per row chunk
constexpr int kMaxGamma = 16;
constexpr int kMaxTreeNodes = 1024;
// Pass-2 workgroups resident per CU (one wave per SIMD each): the second
// launch is sized for this many, and its kernel is built for it.
constexpr int kP2Resident = 6;

// Pass-2 work of a decided sequence.
enum P2Mode : uint32_t {
  P2_NONE = 0,            // output complete after the decision
  P2_RESIDUAL = 1,        // Gumbel-max over ln (p - q)_+ of row `row`
  P2_RESIDUAL_ONEHOT = 2, // Gumbel-max over l/T of row `row`, excluding `x`
  P2_BONUS = 3,           // Gumbel-max over l/T of row gamma
  P2_GREEDY_BONUS = 4     // argmax of row gamma
};

// Per-sequence record in the workspace: one 128-byte line per sequence, so
// that the arrival counters of different sequences never share a line. Zero
// between calls.
struct SeqState {
  uint32_t p2_arrive;  // pass-2 items finished
  uint32_t lbest;      // pass 2: the largest Gumbel total any item of the
                       // sequence has reached so far, as an order key (0: none)
  uint32_t pad0[30];
};
static_assert(sizeof(SeqState) == 128, "one line per sequence");

// Entry of the pass-2 work list: a sequence with a pending draw and its
// decision record, written by its decision item, read by its pass-2 items
// in one round trip:
//   dec[1] = (zt2 bits << 32) | zd2 bits     (log2-domain normalizers)
//   dec[2] = (c2 bits << 32) | invT bits
//   dec[3] = (a_row bits << 32) | x
//   dec[0] = 2^63 | row << 32 | (n + 64) << 8 | mode
//   b      = the sequence
struct WorkRec {
  uint64_t dec[4];
  uint32_t b;
  uint32_t pad[7];
};
static_assert(sizeof(WorkRec) == 64, "half a line per entry");
constexpr uint64_t kRecPublished = 1ull << 63;

// Words of the workspace's control line (ChainArgs::done), on their own
// 128-byte line: sequences appended to the pass-2 work list by the first of two
// launches, and sequences whose pass-2 draw the second launch has finished.
// The last of those returns both to zero.
constexpr int kDoneNWork = 32;
constexpr int kDoneNFinal = 33;

// Pass-1 result of one chunk of one row pair, published as two 64-bit words:
//   sampled:  w0 = (M_target bits << 32) | s_target bits,
//             w1 = (M_draft bits << 32) | s_draft bits  (dense draft), else 1;
//   greedy:   w0 = (max value bits << 32) | (argmax + 1), w1 = 1.
// M is the chunk's largest raw logit and s = sum exp2((l - M) * log2(e) / T)
// (>= 1, so the word is nonzero even when M = +0.0).
struct P1Slot {
  uint64_t w0, w1;
};

// Pass-2 result of one chunk: w0 = (score bits << 32) | index (0xffffffff:
// no candidate), w1 = (residual mass bits << 32) | candidate flag.
struct P2Slot {
  uint64_t w0, w1;
};

// Tree: argmax of one chunk of one node row, (value bits << 32) | (index + 1),
// never zero once written.
typedef uint64_t TreeSlot;

struct ChainArgs {
  const uint8_t* target;
  int64_t t_stride;  // bytes between rows
  const uint8_t* draft;  // NULL: one-hot draft
  int64_t d_stride;
  int32_t d_rows;              // draft rows per sequence: gamma (chains) or N (sampled trees)
  const int32_t* ids;          // [B, gamma]
  const float* temperature;    // [B] or NULL: every sequence greedy
  int32_t B, gamma, V;
  int32_t chunk;    // elements per pass-1 chunk
  int32_t nchunks;  // pass-1 chunks per row
  int32_t kv;       // 16-byte vectors per thread per pass-1 chunk (<= kMaxVecsPerThread)
  int32_t p2_stride;   // pass-2 slots per sequence (>= any chunk count)
  int32_t p2_grid;     // workgroups of the pass-2 launch
  int32_t p2_cap;      // most pass-2 chunks per row
  int32_t p2_force;    // pass-2 chunks per row when > 0 (debug entry point only;
                       // else sized to fill p2_grid)
  int32_t p2_unit;     // pass-2 chunk lengths are multiples of this
  uint32_t key0, key1;
  uint32_t ctr_accept, ctr_noise;  // counter word 3 of the two Philox streams
  uint32_t seq_base;  // counter word 2 of sequence b is seq_base + b
  int32_t* out_tokens;
  int32_t* out_n;
  float* d_accept;
  float* d_logzt;
  float* d_logzd;
  float* d_beta;
  uint32_t* done;     // [64]: [1] nonzero once a bounded wait gave up (the
                      // workspace must then be re-initialized before its next
                      // use); [kDoneNWork], [kDoneNFinal]: the pass-2 work list
  SeqState* seq;      // [B]
  P1Slot* p1;         // [B, gamma, nchunks]
  P2Slot* p2;         // [B, p2_stride]
  WorkRec* work;      // [B] sequences with pass-2 work and their decisions, in
                      // the order the decisions were taken
  uint32_t spin_limit;
};

// Sampled trees (multi-round rejection sampling): the chain arguments with
// gamma = N - 1 (so that target row (b, v) is row b * N + v) and d_rows = N,
// plus the tree. The walk launch gives each sequence W workgroups, each owning
// wlen elements of a row, for the residual-mass passes and the final draw.
struct TreeSampleArgs {
  ChainArgs c;
  const int32_t* parents;  // [N]
  const int32_t* depth;    // [N]
  const int32_t* tokens;   // [B, N]
  int32_t N, max_depth;
  int32_t W, wlen;         // walk: workgroups per sequence, elements per workgroup
  int32_t b_base, b_count; // walk: the sequences of this launch
  P2Slot* slot2;           // walk: the second buffer of workgroup parts, [B, c.p2_stride] (N >= 2)
  int32_t wor;             // siblings drawn without replacement (q renormalized over the tokens not drawn yet)
  int32_t* out_path;       // [B, max_depth + 1]
  int32_t* out_len;        // [B]
  int32_t* out_token;      // [B]
};

struct TreeArgs {
  const uint8_t* target;
  int64_t t_stride;
  const int32_t* parents;
  const int32_t* depth;
  const int32_t* tokens;  // [B, N]
  int32_t B, N, V, max_depth;
  int32_t chunk, nchunks, kv;
  int32_t* out_path;
  int32_t* out_path_len;
  int32_t* out_bonus;
  uint32_t* done;         // as in ChainArgs
  TreeSlot* slot;         // [B, N, nchunks]
  int32_t lag;            // the decision of sequence k follows the items of k + lag
  uint32_t spin_limit;
};

// Block order of a launch that holds both the streaming items (n1 per
// sequence) and the dependent items (n2 per sequence) of m sequences: the
// dependent items of sequence k are placed after the streaming items of
// sequence k + L, so that in the hardware's in-order dispatch they find their
// inputs (nearly always) complete.
struct Layout {
  int m;       // sequences
  int n1, n2;  // items per sequence of each kind
  int L;       // lag
};

// Workgroup id t -> kind (1 streaming, 2 dependent), sequence k, item r.
__device__ __forceinline__ int decode_item(const Layout& q, uint32_t t, int* k, int* r) {
  const uint32_t seg_a = (uint32_t)q.L * q.n1;
  if (t < seg_a) {
    *k = (int)(t / q.n1);
    *r = (int)(t % q.n1);
    return 1;
  }
  t -= seg_a;
  const uint32_t per = (uint32_t)(q.n1 + q.n2);
  const uint32_t seg_b = (uint32_t)(q.m - q.L) * per;
  if (t < seg_b) {
    const int blk = (int)(t / per);
    const int rr = (int)(t % per);
    if (rr < q.n1) {
      *k = q.L + blk;
      *r = rr;
      return 1;
    }
    *k = blk;
    *r = rr - q.n1;
    return 2;
  }
  t -= seg_b;
  *k = (q.m - q.L) + (int)(t / q.n2);
  *r = (int)(t % q.n2);
  return 2;
}

// Workspace carve-up; every offset is a multiple of 256 bytes.
struct WsLayout {
  size_t done, seq, p1, p2, tree_slot, work, total;
};

WsLayout ws_layout(int32_t B, int32_t rows, int32_t nchunks);
int32_t max_chunks(int32_t V);

// Launchers (host). Return hipSuccess or the first HIP error.
hipError_t launch_chain_p1(const ChainArgs& a, bool bf16, bool vec, hipStream_t stream);
hipError_t launch_chain_p2(const ChainArgs& a, bool bf16, bool vec, hipStream_t stream);
hipError_t launch_tree(const TreeArgs& a, bool bf16, bool vec, hipStream_t stream);
int tree_occupancy(bool bf16, bool vec);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
int chain_p2_occupancy(bool bf16, bool vec);
hipError_t launch_tree_sample_walk(const TreeSampleArgs& a, bool bf16, bool vec, hipStream_t stream);
int tree_sample_walk_occupancy(bool bf16, bool vec);

}  // namespace sv
