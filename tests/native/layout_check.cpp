// Host-side check of the index maps in rmx_layout.h, built with g++ under AddressSanitizer
// and UndefinedBehaviorSanitizer (RMX_HD defined empty).  Each map is run over whole buffers
// allocated at exactly the size the library allocates, so an offset past the end is a
// heap-buffer-overflow, and checked against what its documentation states:
//   pk  rows K    packed bf16 layout: a bijection onto pk_rows(rows) x K in 16-byte chunks;
//                 the offset from the block/step/row/chunk description; the producer's
//                 offset equals the byte the matrix-core loop reads; every aligned run of 16
//                 rows reading one chunk index hits 16 distinct 16-byte bank slots
//   mx  rows K    MXFP8 codes (as pk, 64 K per step) and scales: a bijection onto the scale
//                 bytes, and the lane/byte contract of the MFMA scale operand
//   gather        the 16 pieces x 64 lanes of a gathered K step write each LDS slot once,
//                 with the chunk the loop later reads there
//   tiles nMt nNt nblocks   the dense tile order: xcd_remap a bijection of [0, nblocks),
//                 band_tile a bijection onto the nMt x nNt tiles, bands as described
//   moe G nNt maxrows seed zero_pct grid   the Sparse-MoE tile table: moe_tile_locate
//                 inverts the group-by-group numbering; the XCD spans cover every tile once
//   span rows K   the 32-bit descriptor arithmetic of gathered rows does not wrap
// Commands come one per line on stdin; the program prints "ok <line>" per command and exits
// with status 1 at the first failure.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <sstream>
#include <string>
#include <vector>

#include "rmx_layout.h"

using namespace rmx;

static int g_fail = 0;
#define CHECK(cond, ...)                                         \
  do {                                                           \
    if (!(cond)) {                                               \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);  \
      std::fprintf(stderr, __VA_ARGS__);                         \
      std::fprintf(stderr, "\n");                                \
      g_fail = 1;                                                \
      return false;                                              \
    }                                                            \
  } while (0)

// swizzle as described: bits 1 and 2 of the row, exclusive-or'ed, as a 2-bit value
static int swz_desc(int r) { return ((r / 2) ^ (r / 4)) % 4; }

static bool check_pk(int64_t rows, int K) {
  CHECK(K % 32 == 0 && rows > 0, "bad shape");
  const int64_t R = pk_rows(rows);
  CHECK(R % 256 == 0 && R >= rows && R - rows < 256, "pk_rows(%lld) = %lld", (long long)rows, (long long)R);
  const int64_t chunks = R * K / 8;
  unsigned char* hit = new unsigned char[chunks];  // exactly the buffer, in 8-element chunks
  std::memset(hit, 0, chunks);
  const int steps = K / 32;
  for (int64_t row = 0; row < R; ++row) {
    const int r = int(row % 256);
    const int64_t rb = row / 256;
    for (int col = 0; col < K; col += 8) {
      const size_t o = pk_off(int(row), col, K);
      CHECK(o % 8 == 0, "pk_off(%lld, %d) = %zu not chunk-aligned", (long long)row, col, o);
      hit[o / 8] += 1;
      const int kt = col / 32, c = (col / 8) % 4;
      const size_t step_base = size_t(rb * steps + kt) * 8192;  // elements per 256 x 32 step
      const size_t desc = step_base + size_t(r) * 32 + size_t(c ^ swz_desc(r)) * 8;
      CHECK(o == desc, "pk_off(%lld, %d, %d) = %zu, description gives %zu", (long long)row, col, K, o, desc);
      CHECK(2 * o == 2 * step_base + pk_lds_off(r, c), "producer/consumer disagree at row %lld col %d",
            (long long)row, col);
    }
  }
  for (int64_t i = 0; i < chunks; ++i) CHECK(hit[i] == 1, "pk chunk %lld hit %d times", (long long)i, hit[i]);
  delete[] hit;
  // bank slots: 16 consecutive rows (aligned) reading chunk c touch 16 distinct slots of 16 B
  for (int base = 0; base < 256; base += 16)
    for (int c = 0; c < 4; ++c) {
      unsigned seen = 0;
      for (int r = base; r < base + 16; ++r) seen |= 1u << ((pk_lds_off(r, c) % 256) / 16);
      CHECK(seen == 0xffffu, "rows %d..%d chunk %d share bank slots", base, base + 15, c);
    }
  return true;
}

static bool check_mx(int64_t rows, int K) {
  CHECK(K % 64 == 0 && rows > 0, "bad shape");
  const int64_t R = pk_rows(rows);
  const int steps = K / 64;
  const int64_t chunks = R * K / 16;
  unsigned char* hit = new unsigned char[chunks];
  std::memset(hit, 0, chunks);
  const int64_t nscale = R * K / 32;
  unsigned char* shit = new unsigned char[nscale];
  std::memset(shit, 0, nscale);
  for (int64_t row = 0; row < R; ++row) {
    const int r = int(row % 256);
    const int64_t rb = row / 256;
    for (int k = 0; k < K; k += 16) {
      const size_t o = mx_off(int(row), k, K);
      CHECK(o % 16 == 0, "mx_off not chunk-aligned");
      hit[o / 16] += 1;
      const int kt = k / 64, c = (k / 16) % 4;
      const size_t step_base = size_t(rb * steps + kt) * 16384;
      CHECK(o == step_base + size_t(r) * 64 + size_t(c ^ swz_desc(r)) * 16, "mx_off(%lld, %d, %d) = %zu",
            (long long)row, k, K, o);
      CHECK(o == step_base + pk_lds_off(r, c), "mx producer/consumer disagree");
    }
    for (int kb = 0; kb < K / 32; ++kb) shit[mx_scale_off(int(row), kb, K)] += 1;
  }
  for (int64_t i = 0; i < chunks; ++i) CHECK(hit[i] == 1, "mx chunk %lld hit %d times", (long long)i, hit[i]);
  for (int64_t i = 0; i < nscale; ++i) CHECK(shit[i] == 1, "mx scale %lld hit %d times", (long long)i, shit[i]);
  delete[] hit;
  delete[] shit;
  // scale operand: lane l of the wave owning rows 128 h .. of a block reads one 32-bit word
  // at 256 h + 4 l of the step's 512 bytes; its byte i is the scale of row 128 h + 32 i +
  // l % 32 for the 32-value half l / 32 of the step
  for (int64_t rb = 0; rb < R / 256; ++rb)
    for (int kt = 0; kt < steps; ++kt)
      for (int h = 0; h < 2; ++h)
        for (int l = 0; l < 64; ++l)
          for (int i = 0; i < 4; ++i) {
            const int row = int(rb * 256) + 128 * h + 32 * i + l % 32;
            const size_t want = size_t(rb * steps + kt) * 512 + size_t(256 * h + 4 * l + i);
            CHECK(mx_scale_off(row, 2 * kt + l / 32, K) == want, "scale of row %d half %d of step %d", row, l / 32,
                  kt);
          }
  return true;
}

static bool check_gather() {
  unsigned char* slot = new unsigned char[16384 / 16];
  std::memset(slot, 0, 16384 / 16);
  for (int piece = 0; piece < 16; ++piece)
    for (int lane = 0; lane < 64; ++lane) {
      const int row = pk_gather_row(piece, lane);
      CHECK(row >= 0 && row < 256, "gather row %d", row);
      const uint32_t dst = uint32_t(piece * 1024 + lane * 16);
      slot[dst / 16] += 1;
      const int chunk = pk_gather_chunk(row, lane);
      CHECK(chunk >= 0 && chunk < 4, "gather chunk %d", chunk);
      CHECK(pk_lds_off(row, chunk) == dst, "piece %d lane %d: chunk %d of row %d lands at %u, read at %u", piece,
            lane, chunk, row, dst, pk_lds_off(row, chunk));
    }
  for (int i = 0; i < 1024; ++i) CHECK(slot[i] == 1, "LDS slot %d written %d times", i, slot[i]);
  delete[] slot;
  return true;
}

static bool check_tiles(int nMt, int nNt, int nblocks) {
  std::vector<int> seen(static_cast<size_t>(nblocks), 0);
  for (int bid = 0; bid < nblocks; ++bid) {
    const int id = xcd_remap(bid, nblocks);
    CHECK(id >= 0 && id < nblocks, "xcd_remap(%d, %d) = %d", bid, nblocks, id);
    seen[size_t(id)] += 1;
  }
  for (int i = 0; i < nblocks; ++i) CHECK(seen[size_t(i)] == 1, "tile id %d taken %d times", i, seen[size_t(i)]);
  // each XCD (bid % 8) receives a contiguous range of ids, in order
  for (int x = 0; x < NUM_XCD; ++x)
    for (int bid = x; bid + NUM_XCD < nblocks; bid += NUM_XCD)
      CHECK(xcd_remap(bid + NUM_XCD, nblocks) == xcd_remap(bid, nblocks) + 1, "XCD %d range not contiguous", x);
  const int n = nMt * nNt;
  std::vector<int> got(static_cast<size_t>(n), 0);
  int* order = new int[size_t(n)];  // expected: band by band, N tiles, row tiles fastest
  int pos = 0;
  for (int b0 = 0; b0 < nMt; b0 += TILE_BAND)
    for (int nt = 0; nt < nNt; ++nt)
      for (int mt = b0; mt < nMt && mt < b0 + TILE_BAND; ++mt) order[pos++] = mt * nNt + nt;
  CHECK(pos == n, "enumeration");
  for (int rem = 0; rem < n; ++rem) {
    int mt = -1, nt = -1;
    band_tile(rem, nMt, nNt, mt, nt);
    CHECK(mt >= 0 && mt < nMt && nt >= 0 && nt < nNt, "band_tile(%d) = (%d, %d)", rem, mt, nt);
    CHECK(mt * nNt + nt == order[rem], "band_tile(%d, %d, %d) = (%d, %d)", rem, nMt, nNt, mt, nt);
    got[size_t(mt * nNt + nt)] += 1;
  }
  for (int i = 0; i < n; ++i) CHECK(got[size_t(i)] == 1, "tile %d visited %d times", i, got[size_t(i)]);
  delete[] order;
  return true;
}

static bool check_moe(int G, int nNt, int maxrows, unsigned seed, int zero_pct, int grid) {
  std::mt19937 rng(seed);
  std::vector<int> rows(static_cast<size_t>(G));
  for (int g = 0; g < G; ++g)
    rows[size_t(g)] = int(rng() % 100) < zero_pct ? 0 : int(rng() % unsigned(maxrows + 1));
  int* tile_start = new int[size_t(G) + 1];  // exactly the table the route writes
  tile_start[0] = 0;
  for (int g = 0; g < G; ++g) tile_start[g + 1] = tile_start[g] + (rows[size_t(g)] + 255) / 256;
  const int total = tile_start[G] * nNt;
  // expected numbering: group by group, N tile outer, row tile inner
  std::vector<int> eg, emt, ent;
  for (int g = 0; g < G; ++g)
    for (int nt = 0; nt < nNt; ++nt)
      for (int mt = 0; mt < tile_start[g + 1] - tile_start[g]; ++mt) {
        eg.push_back(g);
        ent.push_back(nt);
        emt.push_back(mt);
      }
  CHECK(int(eg.size()) == total, "tile count");
  for (int tile = 0; tile < total; ++tile) {
    int g = -1, mt = -1, nt = -1;
    moe_tile_locate(tile_start, G, nNt, tile, g, mt, nt);
    CHECK(g == eg[size_t(tile)] && mt == emt[size_t(tile)] && nt == ent[size_t(tile)],
          "tile %d: (%d, %d, %d), expected (%d, %d, %d)", tile, g, mt, nt, eg[size_t(tile)], emt[size_t(tile)],
          ent[size_t(tile)]);
    CHECK(rows[size_t(g)] > mt * 256, "tile %d of group %d has no rows", tile, g);
  }
  // persistent grid (a multiple of the XCD count): XCD x takes [lo, hi), its workgroups
  // (blockIdx % 8 == x) stride by grid / 8
  CHECK(grid % NUM_XCD == 0 && grid > 0, "grid");
  const int per_xcd = grid / NUM_XCD;
  std::vector<int> seen(static_cast<size_t>(total), 0);
  for (int bid = 0; bid < grid; ++bid) {
    const int xcd = bid % NUM_XCD, slot_ = bid / NUM_XCD;
    int lo = 0, hi = 0;
    moe_xcd_span(total, xcd, NUM_XCD, lo, hi);
    for (int tile = lo + slot_; tile < hi; tile += per_xcd) {
      CHECK(tile >= 0 && tile < total, "tile %d out of [0, %d)", tile, total);
      seen[size_t(tile)] += 1;
    }
  }
  for (int t = 0; t < total; ++t) CHECK(seen[size_t(t)] == 1, "MoE tile %d run %d times", t, seen[size_t(t)]);
  delete[] tile_start;
  return true;
}

// Gathered rows: offset = row * (2 K) + 16 * chunk + 64 * kt computed in 32 bits, against a
// descriptor of rows * 2 K bytes (rows past the end read as zeros by an offset of exactly
// that size).  The library accepts such an operand only below 2^31 bytes.
static bool check_span(int64_t rows, int K) {
  const uint64_t bytes = uint64_t(rows) * uint64_t(K) * 2u;
  CHECK(bytes < (uint64_t(1) << 31), "operand of %llu bytes is refused by the library", (unsigned long long)bytes);
  const uint32_t row_bytes = uint32_t(K) * 2u, bytesA = uint32_t(rows) * row_bytes;
  CHECK(uint64_t(bytesA) == bytes, "descriptor size wraps");
  const uint32_t last = uint32_t(rows - 1) * row_bytes + 16u * 3u + uint32_t(K / 32 - 1) * 64u + 16u;
  CHECK(uint64_t(last) == uint64_t(rows - 1) * row_bytes + 48 + uint64_t(K / 32 - 1) * 64 + 16, "offset wraps");
  CHECK(last <= bytesA, "last gathered byte %u past %u", last, bytesA);
  return true;
}

int main() {
  std::string line;
  int n = 0;
  char buf[512];
  while (std::fgets(buf, sizeof buf, stdin)) {
    line = buf;
    while (!line.empty() && (line.back() == '\n' || line.back() == '\r')) line.pop_back();
    if (line.empty()) continue;
    std::istringstream in(line);
    std::string cmd;
    in >> cmd;
    bool ok = false;
    if (cmd == "pk") {
      long long r; int K; in >> r >> K; ok = check_pk(r, K);
    } else if (cmd == "mx") {
      long long r; int K; in >> r >> K; ok = check_mx(r, K);
    } else if (cmd == "gather") {
      ok = check_gather();
    } else if (cmd == "tiles") {
      int a, b, c; in >> a >> b >> c; ok = check_tiles(a, b, c);
    } else if (cmd == "moe") {
      int G, nNt, maxrows, zero, grid; unsigned seed;
      in >> G >> nNt >> maxrows >> seed >> zero >> grid;
      ok = check_moe(G, nNt, maxrows, seed, zero, grid);
    } else if (cmd == "span") {
      long long r; int K; in >> r >> K; ok = check_span(r, K);
    } else {
      std::fprintf(stderr, "unknown command: %s\n", line.c_str());
      return 2;
    }
    if (!ok || g_fail) {
      std::fprintf(stderr, "failed: %s\n", line.c_str());
      return 1;
    }
    std::printf("ok %s\n", line.c_str());
    ++n;
  }
  std::printf("%d checks passed\n", n);
  return 0;
}
