// Block metadata of arbitrary dense masks, built on the host.
//
// "hstu_ops.py" (RecML): pointwise_splash_attention turns a numpy array mask
// of shape (q_len, kv_len) into a NumpyMask (then ANDed with the local
// window); the forward walks the non-empty blocks through data_next and, for a
// partial block, fetches that block's mask through a second index map
// (mask_next) into a store of [block_q, block_kv] mask blocks. Equal partial
// blocks share one store entry, which keeps the store small for structured
// masks (every diagonal block of a causal pattern is the same triangle).
//
// Here a block's mask is the dense mask ANDed with the head's band, the
// sequence ends and (when segment ids are given) segment equality, packed as
// bits: row r of entry n is block_kv / 32 words, bit b of word w standing for
// key offset 32 w + b. Classes and data_next follow the same rules as
// splash_mask_info_build (rows, for the forward and the dQ pass) or
// splash_mask_info_build_dkv (columns, for the dK/dV pass; "hstu_ops.py"
// builds the backward's dK/dV mask blocks separately, as
// bwd_mask_info.partial_mask_blocks).

#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "internal.h"

namespace {

using splash::record_error;

}  // namespace

extern "C" splash_status splash_dense_mask_info_host_ex(int B, int q_len, int kv_len, int block_q, int block_kv,
                                                        int num_mask_heads, const splash_head_mask* heads,
                                                        int dense_heads, const uint8_t* dense, int meta_heads,
                                                        const int32_t* q_segment_ids,
                                                        const int32_t* kv_segment_ids, int columns,
                                                        int8_t* block_mask, int32_t* data_next,
                                                        int32_t* mask_next, uint32_t* mask_blocks,
                                                        int64_t capacity, int64_t* num_blocks) {
  if (q_len < 0 || kv_len < 0 || q_len > splash::kMaxLen || kv_len > splash::kMaxLen)
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "bad lengths q_len=%d kv_len=%d", q_len, kv_len);
  if (B < 0 || B > (1 << 24)) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "bad batch B=%d", B);
  if (block_q < 1 || block_q > 1024 || block_kv < 32 || block_kv > 1024 || block_kv % 32 != 0)
    return record_error(SPLASH_ERR_INVALID_ARGUMENT,
                        "block sizes %d x %d: block_q in [1, 1024], block_kv a multiple of 32 in [32, 1024]",
                        block_q, block_kv);
  if (meta_heads < 1 || (num_mask_heads != 1 && num_mask_heads != meta_heads) ||
      (dense_heads != 1 && dense_heads != meta_heads) ||
      meta_heads != (num_mask_heads > dense_heads ? num_mask_heads : dense_heads))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT,
                        "meta_heads=%d must be the larger of num_mask_heads=%d and dense_heads=%d, each 1 or "
                        "meta_heads",
                        meta_heads, num_mask_heads, dense_heads);
  if (heads == nullptr || num_blocks == nullptr)
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "heads and num_blocks must not be null");
  if ((q_segment_ids == nullptr) != (kv_segment_ids == nullptr))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "both or neither of q_segment_ids and kv_segment_ids must be given");
  if (columns != 0 && columns != 1) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "columns=%d must be 0 or 1", columns);
  if (capacity < 0) return record_error(SPLASH_ERR_INVALID_ARGUMENT, "negative capacity");
  const bool seg = q_segment_ids != nullptr;
  const int64_t meta_batch = seg ? B : 1;
  const int64_t nq = (q_len + block_q - 1) / block_q, nk = (kv_len + block_kv - 1) / block_kv;
  const int64_t entries = meta_batch * meta_heads * nq * nk;
  // with all three metadata arrays null the call only counts the store entries
  const bool count_only = block_mask == nullptr && data_next == nullptr && mask_next == nullptr;
  if (entries > 0 && (dense == nullptr || (!count_only && (block_mask == nullptr || data_next == nullptr ||
                                                           mask_next == nullptr))))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "dense mask or an output array is null");
  std::vector<splash::HeadBand> band(num_mask_heads);
  for (int h = 0; h < num_mask_heads; ++h)
    if (!splash::head_band(heads[h], h, &band[h])) return SPLASH_ERR_INVALID_ARGUMENT;

  const int wpr = block_kv / 32;               // words per block row
  const size_t block_words = (size_t)block_q * wpr;
  std::vector<int8_t> cls(entries);
  std::vector<int32_t> nxt(entries), mnext(entries, 0);
  std::vector<uint32_t> store;                 // distinct partial blocks, in first-seen order
  std::unordered_map<std::string, int64_t> index;
  std::vector<uint32_t> bits(block_words);
  // entry of block (i, j) of metadata row-set `base`: rows of kv blocks
  // ([.., nq, nk]) or columns of q blocks ([.., nk, nq])
  auto at = [&](int64_t base, int64_t i, int64_t j) { return base + (columns ? j * nq + i : i * nk + j); };

  for (int64_t bm = 0; bm < meta_batch; ++bm) {
    const int32_t* qs = seg ? q_segment_ids + bm * q_len : nullptr;
    const int32_t* ks = seg ? kv_segment_ids + bm * kv_len : nullptr;
    for (int hm = 0; hm < meta_heads; ++hm) {
      const splash::HeadBand hb = band[num_mask_heads == 1 ? 0 : hm];
      const uint8_t* dm = dense + (dense_heads == 1 ? 0 : (int64_t)hm * q_len * kv_len);
      const int64_t base = (bm * meta_heads + hm) * nq * nk;
      for (int64_t i = 0; i < nq; ++i) {
        for (int64_t j = 0; j < nk; ++j) {
          int64_t count = 0;
          for (int r = 0; r < block_q; ++r) {
            const int64_t q = i * block_q + r;
            for (int w = 0; w < wpr; ++w) {
              uint32_t word = 0;
              if (q < q_len) {
                for (int b = 0; b < 32; ++b) {
                  const int64_t k = j * block_kv + 32 * w + b;
                  const int64_t d = k - q;
                  if (k < kv_len && d >= hb.lo && d <= hb.hi && dm[q * kv_len + k] && (!seg || qs[q] == ks[k]))
                    word |= 1u << b;
                }
              }
              bits[(size_t)r * wpr + w] = word;
              count += __builtin_popcount(word);
            }
          }
          const int8_t c = count == 0 ? 0 : (count == (int64_t)block_q * block_kv ? 2 : 1);
          cls[at(base, i, j)] = c;
          if (c == 1) {
            std::string key(reinterpret_cast<const char*>(bits.data()), block_words * sizeof(uint32_t));
            auto it = index.find(key);
            int64_t n;
            if (it == index.end()) {
              n = (int64_t)(store.size() / block_words);
              index.emplace(std::move(key), n);
              store.insert(store.end(), bits.begin(), bits.end());
            } else {
              n = it->second;
            }
            mnext[at(base, i, j)] = (int32_t)n;
          }
        }
      }
      // data_next: the next non-empty block at or after each position, along
      // kv blocks (rows) or along q blocks (columns); the sentinel is the
      // length of that axis
      const int64_t lines = columns ? nk : nq, len = columns ? nq : nk;
      for (int64_t l = 0; l < lines; ++l) {
        int32_t carry = (int32_t)len;
        for (int64_t x = len - 1; x >= 0; --x) {
          const int64_t e = base + l * len + x;
          if (cls[e] != 0) carry = (int32_t)x;
          nxt[e] = carry;
        }
      }
    }
  }

  const int64_t n = (int64_t)(store.size() / block_words);
  *num_blocks = n;
  if (count_only) return splash::record_ok();
  if (capacity < n || (n > 0 && mask_blocks == nullptr))
    return record_error(SPLASH_ERR_INVALID_ARGUMENT, "mask block capacity %lld < %lld needed", (long long)capacity,
                        (long long)n);
  if (entries > 0) {
    std::memcpy(block_mask, cls.data(), cls.size());
    std::memcpy(data_next, nxt.data(), nxt.size() * sizeof(int32_t));
    std::memcpy(mask_next, mnext.data(), mnext.size() * sizeof(int32_t));
  }
  if (n > 0) std::memcpy(mask_blocks, store.data(), store.size() * sizeof(uint32_t));
  return splash::record_ok();
}

extern "C" splash_status splash_dense_mask_info_host(int q_len, int kv_len, int block_q, int block_kv,
                                                     int num_mask_heads, const splash_head_mask* heads,
                                                     int dense_heads, const uint8_t* dense, int meta_heads,
                                                     int8_t* block_mask, int32_t* data_next, int32_t* mask_next,
                                                     uint32_t* mask_blocks, int64_t capacity,
                                                     int64_t* num_blocks) {
  return splash_dense_mask_info_host_ex(1, q_len, kv_len, block_q, block_kv, num_mask_heads, heads, dense_heads,
                                        dense, meta_heads, nullptr, nullptr, 0, block_mask, data_next, mask_next,
                                        mask_blocks, capacity, num_blocks);
}
