// qsa_internal.h — argument blocks and launchers shared by the ABI layer (qsa_api.cpp) and
// the kernels (qsa_kernels.hip, qsa_scores.hip, qsa_select.hip, qsa_copy.hip).  Not part of
// the public ABI, which is include/qsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

enum class Dt : int { F16 = 0, BF16 = 1 };

// Pool addressing of the page's QsaIndexerPoolState, pre-digested on the host.
struct PoolArgs {
  void* base;               // T [2*numPages, 128, H, D]
  const int32_t* pageTable; // int32 [B, 2, maxPagesPerSeq]
  int32_t maxPagesPerSeq;
  int32_t numIds;           // 2*numPages: valid ids are [0, numIds)
  int64_t rowElems;         // H*D: elements per pool row
  int32_t headSize;         // first indexer column (head 0)
};

// Per-sequence block triplet source: scalars, or three device arrays.
struct Ranges {
  int32_t blockBegin, blockEnd, pastLen;  // scalar mode
  const int32_t* pastLens;                // non-null: ranges mode
  const int32_t* blockBegins;
  const int32_t* blockEnds;
  int32_t span;                           // blocks per sequence the grid covers
};

struct QPrepArgs {
  void* qNormed;
  const void* indexQk;
  const float* cosSin;
  const int32_t* ctx;
  const void* wQ;
  float eps;
  int32_t B, S;
  float* dMeanSq;  // debug outputs (debug kernels only)
  float* dInv;
  float* dPre;
};

struct KCompressArgs {
  void* kbar;
  const void* indexQk;
  const float* cosSin;
  int32_t maxPositions;
  const int32_t* ctx;
  const void* wK;
  float eps;
  int32_t B, S, numBlocks;
  Ranges r;
  PoolArgs pool;  // base == nullptr: no V-tail write
  void* dMT;      // debug outputs (debug kernels only)
  float* dMeanSq;
  float* dInv;
  float* dPre;
};

struct PersistArgs {
  PoolArgs pool;
  const void* indexQk;
  const void* kbar;  // nullptr: raw-K tails only
  const int32_t* ctx;
  int32_t B, S, numBlocks;
  Ranges r;
};

struct PrefillArgs {
  void* qNormed;
  void* kbar;
  const void* indexQk;
  const float* cosSin;
  const int32_t* ctx;
  const void* wQ;
  const void* wK;
  float eps;
  int32_t B, S, numBlocks;
  PoolArgs pool;  // base == nullptr: no pool writes
};

struct PreDecodeArgs {
  void* qNormed;
  const void* indexQk;
  const float* cosSin;
  int32_t maxPositions;
  const int32_t* ctx;
  const int32_t* newLens;  // nullptr: one new token per sequence
  const void* wQ;
  const void* wK;
  float eps;
  int32_t B, S;
  PoolArgs pool;
};

// Block scores over global rows [rowStart, rowStart + numRows).  The launcher fills the tile
// fields: workgroup tiles of consecutive tokens of one sequence, numTiles of them starting at
// tile0 (tile = b * tilesPerSeq + t / tokens per tile).
struct ScoresArgs {
  float* logits;
  const void* qNormed;
  const void* kbar;
  const int32_t* ctx;
  int32_t B, S, numBlocks;
  int64_t rowStart, numRows;
  int64_t tile0, tilesPerSeq, numTiles;
};

struct ScoresDecodeArgs {
  float* logits;
  const void* qNormed;
  const int32_t* ctx;
  PoolArgs pool;
  int32_t B, maxBlocks;
};

// K4 over rows [rowStart, rowStart + numRows); sortedIds is [numRows, numBlocks].
struct ExpandArgs {
  int32_t* outIdx;
  const int32_t* sortedIds;
  const int32_t* ctx;
  int32_t S, numBlocks;
  int64_t rowStart, numRows;
};

// Prefill selection + K4 over rows [rowStart, rowStart + numRows); logits is [numRows, numBlocks].
struct TopkArgs {
  int32_t* outIdx;
  const float* logits;
  const int32_t* ctx;
  int32_t S, numBlocks;
  int64_t rowStart, numRows;
};

struct TopkDecodeArgs {
  int32_t* outIdx;
  const float* logits;
  const int32_t* ctx;
  int32_t* splitCounters;  // nullable: [B, numKVHeads] zeroed
  int32_t numKVHeads;
  int32_t B, maxBlocks;
  int32_t chunk = 0, numChunks = 0;  // split rows: set by the launcher
};

// Launchers: enqueue on `stream`, return the launch status.  Arguments are already validated.
hipError_t launch_q_prep(const QPrepArgs& a, Dt dt, bool debug, hipStream_t stream);
hipError_t launch_k_compress(const KCompressArgs& a, Dt dt, bool debug, hipStream_t stream);
hipError_t launch_persist(const PersistArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, Dt dt, hipStream_t stream);
hipError_t launch_pre_decode(const PreDecodeArgs& a, Dt dt, hipStream_t stream);
hipError_t launch_scores(const ScoresArgs& a, Dt dt, hipStream_t stream);
// Workgroups of the prefill scores launch for a.S, a.numBlocks, a.rowStart, a.numRows (the
// launcher fills the tile fields the same way), and its threads per workgroup.
int64_t scores_workgroups(ScoresArgs& a);
// Workgroups (64 threads) of the decode scores launch for B sequences of maxBlocks blocks.
int64_t scores_decode_workgroups(int32_t B, int32_t maxBlocks);
// Workgroups of the largest grid the decode selection launches for B sequences of maxBlocks.
int64_t topk_decode_workgroups(int32_t B, int32_t maxBlocks);
constexpr int kScoresThreads = 512;
hipError_t launch_scores_decode(const ScoresDecodeArgs& a, Dt dt, hipStream_t stream);
hipError_t launch_ids_fill(int32_t* ids, int64_t total, int32_t numBlocks, hipStream_t stream);

// Plain copy of `bytes` (a multiple of 16; both pointers 16-byte aligned).
hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);
hipError_t launch_expand(const ExpandArgs& a, hipStream_t stream);
hipError_t launch_topk_expand(const TopkArgs& a, hipStream_t stream);
hipError_t launch_topk_expand_decode(const TopkDecodeArgs& a, hipStream_t stream);

}  // namespace qsa
