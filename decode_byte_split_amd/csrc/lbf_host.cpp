// lbf_host.cpp — host-side helpers of the entropy-coded (K15H) variant that
// involve no GPU code: Huffman code lengths, canonical codes and the blob
// layout.  Kept apart from the kernels so that every piece of host logic of
// the library builds as plain C++ (the CPU sanitizer test compiles it so).
// The variant entropy-codes the per-weight exponent codes while sign and
// mantissa stay raw, as DFloat11 does ("你的 bf16 模型,有 5 個 bit 是廢的",
// section 二); the procedure and its tie rule are in include/lbf.h (K15H).
#include <algorithm>
#include <utility>
#include <vector>

#include "lbf.h"
#include "lbf_internal.h"

namespace lbf {

// Huffman code lengths (see include/lbf.h for the procedure and its tie rule).
// Leaves, then merged nodes, live in one array; each merge records its two
// children, and lengths are the depths found walking down from the root.
void huffman_lengths(const uint64_t count[16], uint8_t len[16]) {
  std::fill(len, len + 16, (uint8_t)0);
  std::vector<int> sym;
  for (int s = 0; s < 16; s++)
    if (count[s]) sym.push_back(s);
  std::stable_sort(sym.begin(), sym.end(), [&](int a, int b) { return count[a] < count[b]; });
  const int m = (int)sym.size();
  if (m == 0) return;
  if (m == 1) {
    len[sym[0]] = 1;
    return;
  }
  struct Node {
    uint64_t weight;
    int child[2];  // -1 for a leaf
  };
  std::vector<Node> node;
  for (int s : sym) node.push_back(Node{count[s], {-1, -1}});
  size_t leaf = 0, merged = (size_t)m;  // fronts of the two queues
  while (node.size() < (size_t)(2 * m - 1)) {
    int take[2];
    for (int k = 0; k < 2; k++) {
      const bool use_leaf = leaf < (size_t)m && (merged >= node.size() || node[leaf].weight <= node[merged].weight);
      take[k] = (int)(use_leaf ? leaf++ : merged++);
    }
    node.push_back(Node{node[take[0]].weight + node[take[1]].weight, {take[0], take[1]}});
  }
  std::vector<std::pair<int, int>> stack{{(int)node.size() - 1, 0}};
  while (!stack.empty()) {
    const auto [id, depth] = stack.back();
    stack.pop_back();
    if (node[id].child[0] < 0) {
      len[sym[id]] = (uint8_t)depth;
    } else {
      stack.push_back({node[id].child[0], depth + 1});
      stack.push_back({node[id].child[1], depth + 1});
    }
  }
}

// Canonical codes, reversed for the least-significant-bit-first stream:
// symbols in (length, symbol) order take consecutive values, the value
// doubling (shifting left) whenever the length grows.
HCode hcode_of(const uint8_t len[16]) {
  HCode h{};
  std::vector<int> order;
  for (int s = 0; s < 16; s++)
    if (len[s]) order.push_back(s);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return len[a] < len[b]; });
  uint32_t code = 0, prev = 0;
  for (int s : order) {
    code <<= (len[s] - prev);
    prev = len[s];
    uint32_t rev = 0;
    for (uint32_t b = 0; b < len[s]; b++) rev |= ((code >> b) & 1u) << (len[s] - 1 - b);
    h.sym[s] = rev << 4 | len[s];
    code++;
  }
  return h;
}

HLayout hlayout_of(uint64_t rows, uint64_t cols, uint64_t n_esc, uint64_t stream_words) {
  auto up = [](uint64_t v) { return (v + 255) & ~uint64_t(255); };
  HLayout L;
  L.n = rows * cols;
  L.n_tiles = (L.n + LBF_TILE - 1) / LBF_TILE;
  L.n_esc = n_esc;
  L.stream_words = stream_words;
  L.off_raw = LBF_HEADER_BYTES;
  L.off_bits = up(L.off_raw + L.n_tiles * LBF_TILE);
  L.off_woff = up(L.off_bits + 4 * stream_words);
  L.off_idx = up(L.off_woff + 4 * (L.n_tiles + 1));
  L.off_esc = up(L.off_idx + 4 * (L.n_tiles + 1));
  L.blob_bytes = up(L.off_esc + n_esc);
  return L;
}

}  // namespace lbf
