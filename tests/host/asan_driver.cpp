// CPU driver for the library's host-only unit (host_checks.cpp), built with
// the address and undefined-behaviour sanitizers by test_host_sanitize.py.
//
// Reads one case per line on stdin and prints one result line per case:
//   fwd_bwd X W t s BT H V C dt loss rl dX dW ws wsb err  -> status of check_fwd_bwd
//   fwd X W t BT H V C dt loss rl ws wsb err              -> status of check_fwd
//   orpo X W t ns T H V C dt loss sl dX dW ws wsb err     -> status of check_orpo
//   ce lg t BT V loss rl ws wsb err                       -> status of check_ce
//   ce_noalloc lg t BT V loss rl err max_rows             -> status of check_ce_noalloc
//   layout BT H V C dt                                    -> "ok" or the broken layout invariant
//   query BT H V C dt                                     -> the size queries of flce.h, comma-separated
//   tiles N                                               -> "ok" or the broken invariant of the per-XCD tile
//                                                            ranges, for every launch of 0 .. N tiles
// Pointers are plain integers (never dereferenced); 0 is a null pointer.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "../../include/flce.h"
#include "../../linear_cross_entropy_05_amd/csrc/flce_host.h"

namespace {

const void* P(unsigned long long v) { return reinterpret_cast<const void*>((uintptr_t)v); }
template <typename T>
const T* PT(unsigned long long v) {
  return reinterpret_cast<const T*>((uintptr_t)v);
}

bool a256(size_t x) { return (x & 255) == 0; }

// Invariants of the forward+backward layout: 256-byte aligned, disjoint
// regions in order, each large enough for what the kernels put there.
std::string check_layout(const flce::Layout& L, int64_t BT, int64_t H, int64_t V, int64_t C_req) {
  const size_t es = (size_t)L.esize;
  if (L.ldz % flce::kTile || L.ldz < V || L.nvt * flce::kTile != L.ldz) return "ldz/nvt";
  if (L.C < 1 || (BT > 0 && L.C > BT)) return "chunk range";
  if (C_req <= 0 && BT > 0 && L.C > flce::kTile && (size_t)L.C * L.ldz * es > ((size_t)1 << 30))
    return "chunk above 1 GiB";
  if (L.splits < 1 || L.splits > 16) return "splits";
  if (L.ldxt < L.C || L.ldxt % 64) return "ldxt";
  const size_t offs[] = {L.off_nvalid, L.off_lse, L.off_rowloss, L.off_part, L.off_chunk, L.off_dxpart, L.total};
  for (size_t o : offs)
    if (!a256(o)) return "unaligned offset";
  if (L.off_nvalid + 16 > L.off_queue || L.off_queue % 16 || L.off_queue + 32 > L.off_lse) return "nvalid/queue region";
  if (L.off_lse + (size_t)L.C * 4 > L.off_rowloss) return "lse region";
  if (L.compact) {
    const size_t coffs[] = {L.off_idx, L.off_ys, L.off_ss, L.off_xs};
    for (size_t o : coffs)
      if (!a256(o)) return "unaligned compaction offset";
    if (L.off_rowloss + (size_t)(BT > 0 ? BT : 1) * 4 > L.off_idx) return "rowloss region";
    if (L.off_idx + (size_t)(BT > 0 ? BT : 1) * 4 > L.off_ys) return "idx region";
    if (L.off_ys + (size_t)L.C * 8 > L.off_ss) return "ys region";
    if (L.off_ss + (size_t)L.C * 4 > L.off_xs) return "ss region";
    if (L.off_xs + (size_t)L.C * H * es > L.off_part) return "xs region";
  } else {
    if (L.off_idx || L.off_ys || L.off_ss || L.off_xs) return "compaction regions without compaction";
    if (L.off_rowloss + (size_t)(BT > 0 ? BT : 1) * 4 > L.off_part) return "rowloss region";
  }
  const size_t stats = (size_t)L.C * 2 * L.nvt * 8;
  const size_t xt = L.dtype == FLCE_BF16 ? (size_t)H * L.ldxt * 2 : 0;
  if (L.off_part + stats > L.off_chunk || L.off_part + xt > L.off_chunk) return "statistics region";
  if (L.off_chunk + (size_t)L.C * L.ldz * es > L.off_dxpart) return "chunk region";
  if (L.splits > 1 && L.off_dxpart + (size_t)L.splits * L.C * H * 4 > L.total) return "dx partials region";
  if (L.off_dxpart > L.total) return "total";
  return "ok";
}

std::string check_fwd_layout(const flce::Layout& L, int64_t BT) {
  const size_t offs[] = {L.off_nvalid, L.off_lse, L.off_rowloss, L.off_part, L.off_chunk, L.total};
  for (size_t o : offs)
    if (!a256(o)) return "fwd unaligned offset";
  if (L.C < 1 || (BT > 0 && L.C > BT)) return "fwd pass range";
  if (L.off_nvalid + 16 > L.off_queue || L.off_queue % 16 || L.off_queue + 32 > L.off_lse) return "fwd nvalid/queue region";
  if (L.off_lse + (size_t)L.C * 4 > L.off_rowloss) return "fwd lse region";
  if (L.off_rowloss + (size_t)(BT > 0 ? BT : 1) * 4 > L.off_part) return "fwd rowloss region";
  if (L.off_part + (size_t)L.C * 2 * L.nvt * 8 > L.total) return "fwd statistics region";
  if (L.off_chunk != L.total || L.off_dxpart != L.total) return "fwd has a chunk";
  return "ok";
}

// The per-XCD ranges of a launch of `total` items partition [0, total) in
// order, differ in length by at most one, and a queue launch gives every XCD
// at least as many workgroups as its range.
std::string check_tiles(int64_t total) {
  int64_t next = 0, lmin = total, lmax = 0;
  for (int x = 0; x < flce::kXcds; ++x) {
    const int64_t f = flce::xcd_first(total, x), l = flce::xcd_len(total, x);
    if (f != next || l < 0) return "ranges not contiguous";
    next = f + l;
    lmin = l < lmin ? l : lmin;
    lmax = l > lmax ? l : lmax;
    if (flce::queue_grid(total) / flce::kXcds < l) return "queue grid short";
  }
  if (next != total) return "ranges do not cover the launch";
  if (lmax - lmin > 1) return "ranges unbalanced";
  if (flce::queue_grid(total) % flce::kXcds) return "queue grid not a multiple of the XCDs";
  return "ok";
}

// Two kinds of items in one launch (n0 then n1 per XCD range): every item of
// each kind is at exactly one (XCD, position), kind 0 before kind 1 within a
// range, nothing past the range, and the queue grid covers each range.
std::string check_items(int64_t n0, int64_t n1) {
  std::string seen0((size_t)n0, '0'), seen1((size_t)n1, '0');
  for (int y = 0; y < flce::kXcds; ++y) {
    const int64_t len = flce::xcd_len(n0, y) + flce::xcd_len(n1, y);
    if (flce::queue_grid(n0 + n1) / flce::kXcds < len) return "queue grid short for two kinds";
    int last_kind = 0;
    for (int64_t v = 0; v < len; ++v) {
      const flce::XcdItem it = flce::xcd_item(n0, n1, y, v);
      if (it.kind < last_kind) return "kind 1 before kind 0";
      last_kind = it.kind;
      std::string& seen = it.kind ? seen1 : seen0;
      const int64_t n = it.kind ? n1 : n0;
      if (it.item < 0 || it.item >= n || seen[(size_t)it.item] != '0') return "item map not a bijection";
      seen[(size_t)it.item] = '1';
    }
    if (flce::xcd_item(n0, n1, y, len).item != -1) return "item past the range";
  }
  if (seen0.find('0') != std::string::npos || seen1.find('0') != std::string::npos) return "item never taken";
  return "ok";
}

}  // namespace

int main() {
  char line[1024];
  while (fgets(line, sizeof line, stdin)) {
    char op[32];
    if (sscanf(line, "%31s", op) != 1) continue;
    unsigned long long X, W, t, s, loss, rl, dX, dW, ws, wsb, err, lg, sl;
    long long BT, H, V, C, ns, T;
    int dt;
    if (!strcmp(op, "fwd_bwd") &&
        sscanf(line, "%*s %llu %llu %llu %llu %lld %lld %lld %lld %d %llu %llu %llu %llu %llu %llu %llu", &X, &W, &t,
               &s, &BT, &H, &V, &C, &dt, &loss, &rl, &dX, &dW, &ws, &wsb, &err) == 16) {
      flce::Layout L;
      printf("%d\n", flce::check_fwd_bwd(P(X), P(W), PT<int64_t>(t), PT<float>(s), BT, H, V, C, dt, PT<float>(loss),
                                         PT<float>(rl), P(dX), PT<float>(dW), P(ws), (size_t)wsb, PT<int32_t>(err),
                                         &L));
    } else if (!strcmp(op, "fwd") &&
               sscanf(line, "%*s %llu %llu %llu %lld %lld %lld %lld %d %llu %llu %llu %llu %llu", &X, &W, &t, &BT, &H,
                      &V, &C, &dt, &loss, &rl, &ws, &wsb, &err) == 13) {
      flce::Layout L;
      printf("%d\n", flce::check_fwd(P(X), P(W), PT<int64_t>(t), BT, H, V, C, dt, PT<float>(loss), PT<float>(rl),
                                     P(ws), (size_t)wsb, PT<int32_t>(err), &L));
    } else if (!strcmp(op, "orpo") &&
               sscanf(line, "%*s %llu %llu %llu %lld %lld %lld %lld %lld %d %llu %llu %llu %llu %llu %llu %llu", &X, &W,
                      &t, &ns, &T, &H, &V, &C, &dt, &loss, &sl, &dX, &dW, &ws, &wsb, &err) == 16) {
      flce::OrpoLayout L;
      printf("%d\n", flce::check_orpo(P(X), P(W), PT<int64_t>(t), ns, T, H, V, C, dt, PT<float>(loss), PT<float>(sl),
                                      P(dX), PT<float>(dW), P(ws), (size_t)wsb, PT<int32_t>(err), &L));
    } else if (!strcmp(op, "ce") && sscanf(line, "%*s %llu %llu %lld %lld %llu %llu %llu %llu %llu", &lg, &t, &BT, &V,
                                           &loss, &rl, &ws, &wsb, &err) == 9) {
      printf("%d\n", flce::check_ce(PT<float>(lg), PT<int64_t>(t), BT, V, PT<float>(loss), PT<float>(rl), P(ws),
                                    (size_t)wsb, PT<int32_t>(err)));
    } else if (!strcmp(op, "ce_noalloc") && sscanf(line, "%*s %llu %llu %lld %lld %llu %llu %llu %lld", &lg, &t, &BT,
                                                  &V, &loss, &rl, &err, &C) == 8) {
      printf("%d\n", flce::check_ce_noalloc(PT<float>(lg), PT<int64_t>(t), BT, V, PT<float>(loss), PT<float>(rl),
                                            PT<int32_t>(err), C));
    } else if (!strcmp(op, "layout") && sscanf(line, "%*s %lld %lld %lld %lld %d", &BT, &H, &V, &C, &dt) == 5) {
      std::string r = check_layout(flce::make_layout(BT, H, V, C, dt, true), BT, H, V, C);
      if (r == "ok") r = check_layout(flce::make_layout(BT, H, V, C, dt, false), BT, H, V, C);
      if (r == "ok") r = check_fwd_layout(flce::make_fwd_layout(BT, H, V, C, dt), BT);
      for (int ns = 2; r == "ok" && ns <= 8; ns += 6) {
        if (BT < ns || BT % ns) continue;
        const int64_t T = BT / ns, B = ns / 2;
        const flce::OrpoLayout O = flce::make_orpo_layout(ns, T, H, V, C, dt);
        if (O.one_pass) {
          const size_t es = dt == 1 ? 2 : 4;
          if (O.pairs < 1 || O.pairs > B || O.Cp != 2 * O.pairs * T || O.Cp > flce::make_layout(BT, H, V, C, dt, false).C)
            r = "orpo pairs per chunk";
          else if (O.off_nvalid + 12 > O.off_rlc || O.off_rlc + (size_t)O.Cp * 4 > O.off_wc ||
                   O.off_wc + (size_t)O.Cp * 4 > O.off_seq || O.off_seq + (size_t)ns * 24 > O.off_pair ||
                   O.off_pair + (size_t)B * 8 > O.off_xg || O.off_xg + (size_t)O.Cp * H * es > O.off_yg ||
                   O.off_yg + (size_t)O.Cp * 8 > O.off_dxc || O.off_dxc + (size_t)O.Cp * H * es > O.off_region ||
                   O.off_region + O.fb.total != O.total || !a256(O.off_region) || O.fb.C != O.Cp || O.fb.compact)
            r = "orpo one-pass layout";
        } else {
          const size_t region = O.fwd.total > O.fb.total ? O.fwd.total : O.fb.total;
          if (O.off_region + region != O.total || !a256(O.off_region) || O.fb.compact ||
              O.off_scale + (size_t)BT * 4 > O.off_scratch || O.off_rowloss + (size_t)BT * 4 > O.off_scale)
            r = "orpo layout";
        }
      }
      if (r == "ok" && flce_workspace_bytes(BT, H, V, C, dt) != (BT < 0 ? 0 : flce::make_layout(BT, H, V, C, dt, true).total))
        r = "workspace query";
      printf("%s\n", r.c_str());
    } else if (!strcmp(op, "tiles") && sscanf(line, "%*s %lld", &BT) == 1) {
      std::string r = "ok";
      for (int64_t n = 0; n <= BT && r == "ok"; ++n) r = check_tiles(n);
      for (int64_t n : {(int64_t)8016, (int64_t)16032, (int64_t)(1 << 30) - 1, (int64_t)(1 << 30)})
        if (r == "ok") r = check_tiles(n);
      // dX items then dW tiles: small sizes exhaustively, then the heads' shapes
      for (int64_t a = 0; a <= 40 && r == "ok"; ++a)
        for (int64_t b = 0; b <= 40 && r == "ok"; ++b) r = check_items(a, b);
      for (int64_t a : {(int64_t)240, (int64_t)256, (int64_t)1274, (int64_t)768})
        for (int64_t b : {(int64_t)8016, (int64_t)8316, (int64_t)12000, (int64_t)1000})
          if (r == "ok") r = check_items(a, b);
      printf("%s\n", r.c_str());
    } else if (!strcmp(op, "query") && sscanf(line, "%*s %lld %lld %lld %lld %d", &BT, &H, &V, &C, &dt) == 5) {
      printf("%lld,%zu,%zu,%zu,%zu\n", (long long)flce_chunk_tokens(BT, H, V, C, dt),
             flce_workspace_bytes(BT, H, V, C, dt), flce_fwd_workspace_bytes(BT, H, V, C, dt),
             flce_orpo_workspace_bytes(2, BT, H, V, C, dt), ce_workspace_bytes(BT, V));
    } else {
      printf("bad line\n");
    }
    fflush(stdout);
  }
  return 0;
}
