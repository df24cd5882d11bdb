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

// Pass-2 work of a decided sequence.
enum P2Mode : uint32_t {
  P2_NONE = 0,            // output complete after the decision
  P2_RESIDUAL = 1,        // Gumbel-max over ln (p - q)_+ of row `row`
  P2_RESIDUAL_ONEHOT = 2, // Gumbel-max over l/T of row `row`, excluding `x`
  P2_BONUS = 3,           // Gumbel-max over l/T of row gamma
  P2_GREEDY_BONUS = 4     // argmax of row gamma
};

// Per-sequence record in the workspace (64 bytes). Zero between calls.
struct SeqState {
  uint32_t p2_arrive;  // pass-2 items finished
  uint32_t pad[15];
};

// Pass-1 result of one chunk of one row pair, published as two 64-bit words
// that are never zero once written (so a reader can wait for them):
//   sampled:  w0 = (M_target bits << 32) | s_target bits,
//             w1 = (M_draft bits << 32) | s_draft bits  (dense draft) or 1;
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

struct TreePartial {
  float v;
  int32_t i;
};

struct ChainArgs {
  const uint8_t* target;
  int64_t t_stride;  // bytes between rows
  const uint8_t* draft;  // NULL: one-hot draft
  int64_t d_stride;
  const int32_t* ids;          // [B, gamma]
  const float* temperature;    // [B] or NULL: every sequence greedy
  int32_t B, gamma, V;
  int32_t chunk;    // elements per pass-1 chunk
  int32_t nchunks;  // pass-1 chunks per row
  int32_t kv;       // 16-byte vectors per thread per pass-1 chunk (<= kMaxVecsPerThread)
  int32_t p2_chunk;    // elements per pass-2 chunk
  int32_t p2_nchunks;  // pass-2 chunks per row
  uint32_t key0, key1;
  uint32_t ctr_accept, ctr_noise;  // counter word 3 of the two Philox streams
  int32_t* out_tokens;
  int32_t* out_n;
  float* d_accept;
  float* d_logzt;
  float* d_logzd;
  float* d_beta;
  uint32_t* done;     // [1]: nonzero once a bounded wait of a call gave up (sticky)
  SeqState* seq;      // [B]
  P1Slot* p1;         // [B, gamma, nchunks]
  P2Slot* p2;         // [B, p2_nchunks]
  int32_t lag;        // pass-2 items of sequence k follow the pass-1 items of k + lag
  int32_t fused;      // one launch for both passes
  uint32_t spin_limit;
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
  uint32_t* arrive;       // [B]
  TreePartial* part;      // [B, N, nchunks]
};

// Workspace carve-up; every offset is a multiple of 256 bytes.
struct WsLayout {
  size_t done, seq, p1, p2, tree_arrive, tree_part, total;
};

WsLayout ws_layout(int32_t B, int32_t rows, int32_t nchunks);
int32_t max_chunks(int32_t V);

// Launchers (host). Return hipSuccess or the first HIP error.
hipError_t launch_chain(const ChainArgs& a, bool bf16, bool vec, hipStream_t stream);
hipError_t launch_chain_p1(const ChainArgs& a, bool bf16, bool vec, hipStream_t stream);
hipError_t launch_chain_p2(const ChainArgs& a, bool bf16, bool vec, hipStream_t stream);
hipError_t launch_tree(const TreeArgs& a, bool bf16, bool vec, hipStream_t stream);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
int chain_occupancy(bool bf16, bool vec);

}  // namespace sv
