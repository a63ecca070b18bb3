// Workspace layouts and split counts of the libkvq kernels: plain host
// arithmetic, kept apart from the kernels so that the host side of the
// library (validation, tables, layouts) also builds and runs without a GPU.
#include "kvq_internal.h"

namespace kvq {

size_t decode_count_bytes(int64_t B_Hkv) { return ((size_t)B_Hkv * sizeof(uint32_t) + 255) / 256 * 256; }

// Decode: arrival counters [B H_kv] (decode_count_bytes), split partials
// [B H_q][max splits][2 + 128] fp32, then the dense rotation's rotated
// queries [B H_q][128] fp32.
size_t decode_ws_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t T)
{
    const int64_t bhs = B * Hkv;
    const int64_t max_split = decode_max_splits(T);
    return decode_count_bytes(bhs) +
           (size_t)(B * Hq) * (size_t)max_split * (kD + 2) * sizeof(float) + (size_t)(B * Hq) * kD * sizeof(float);
}

int decode_auto_splits(int64_t B, int64_t Hkv, int64_t T)
{
    // about one block (16 waves) per compute unit, and at least 1024 tokens per block
    const int64_t bhs = B * Hkv;
    int64_t ns = (256 + bhs - 1) / bhs;
    const int64_t cap = (T + 1023) / 1024;
    if (ns > cap) ns = cap;
    return (int)(ns < 1 ? 1 : ns);
}

// The no-allocation scratch: a fixed counter region (kNoAllocCountBytes),
// then the layout above with exactly n_split partial slots per (batch, query
// head); SIZE_MAX when the counters of B H_kv groups do not fit their region.
size_t noalloc_decode_bytes(int64_t B, int64_t Hq, int64_t Hkv, int n_split, bool dense)
{
    const int64_t bhs = B * Hkv;
    if (decode_count_bytes(bhs) > kNoAllocCountBytes) return SIZE_MAX;
    return kNoAllocCountBytes +
           (size_t)(B * Hq) * (size_t)n_split * (kD + 2) * sizeof(float) +
           (dense ? (size_t)(B * Hq) * kD * sizeof(float) : 0);
}

// NSN statistics: channel sums per (head, 2048-token chunk), fp32 [H][chunks][128].
size_t nsn_ws_bytes(int64_t H, int64_t T)
{
    const int64_t n_chunks = (T + kNsnChunk - 1) / kNsnChunk;
    return (size_t)H * n_chunks * kD * sizeof(float);
}

size_t nsn_ws_bytes_aligned(int64_t H, int64_t T) { return (nsn_ws_bytes(H, T) + 255) / 256 * 256; }

// Double quantisation: the dequantised means [H][128] fp32 after the sums.
size_t nsn_dq_ws_bytes(int64_t H, int64_t T) { return nsn_ws_bytes_aligned(H, T) + (size_t)H * kD * sizeof(float); }

// NSN-VQ decode: tokens per split (a multiple of the 64-token tile), the
// automatic split count (about one block per compute unit), and the partials
// [B H_q][max splits][kNsnPartStride] fp32.
int64_t nsn_decode_chunk(int64_t T, int n_split)
{
    const int64_t per = (T + n_split - 1) / n_split;
    return (per + 63) / 64 * 64;
}

int nsn_decode_auto_splits(const kvq_ctx *ctx, int64_t B, int64_t T)
{
    const int64_t groups = B * ctx->H;
    int64_t ns = (ctx->n_cu + groups - 1) / groups;
    const int64_t cap = decode_max_splits(T);
    if (ns > cap) ns = cap;
    return ns < 1 ? 1 : (int)ns;
}

size_t nsn_decode_ws_bytes(int64_t B, int64_t Hq, int64_t T)
{
    return (size_t)B * Hq * decode_max_splits(T) * kNsnPartStride * sizeof(float);
}

// Streaming NSN-VQ decode: splits hold whole flush groups (Gs tokens, a
// multiple of 64) and at most kNsnMaxGroupsBlk of them; one partial slot per
// split (at most kMaxSplits - 1) plus the window's.
int64_t nsn_stream_chunk(int64_t T, int n_split, int64_t Gs)
{
    const int64_t per = (T + n_split - 1) / n_split;
    int64_t chunk = (per + Gs - 1) / Gs * Gs;
    if (chunk > kNsnMaxGroupsBlk * Gs) chunk = kNsnMaxGroupsBlk * Gs;
    if ((T + chunk - 1) / chunk > kMaxSplits - 1) return 0;
    return chunk;
}

size_t nsn_stream_ws_bytes(int64_t B, int64_t Hq, int64_t T_cap)
{
    int64_t slots = (T_cap + 63) / 64;
    if (slots > kMaxSplits - 1) slots = kMaxSplits - 1;
    return (size_t)B * Hq * (slots + 1) * kNsnPartStride * sizeof(float);
}

}  // namespace kvq
