// pool_replay.cpp -- a host-only driver of the page table (csrc/pool.cpp) for
// the sanitizer test: it reads one operation per line from stdin, runs it
// through the C ABI and prints one result line, so a test can compare the
// results with the page-pool model and let AddressSanitizer /
// UndefinedBehaviorSanitizer watch every step.  Built by the test with g++
// (no GPU code is involved), never shipped in the library.
//
//   create N P FLAGS            -> create <status>
//   begin ID n t1 .. tn         -> begin <status> <cached_len>
//   append ID n t1 .. tn        -> append <status>
//   reserve ID n                -> reserve <status> [slots...]
//   commit ID n                 -> commit <status>
//   bt ID                       -> bt <status> [pages...]
//   len ID                      -> len <value>
//   end ID                      -> end <status>
//   evict W                     -> evict <status> <evicted>
//   pages                       -> pages <free> <refs:published for every page>
//   vslots n s1 .. sn           -> vslots <status>   (ia_validate_slots with the pool)
#include <cstdarg>
#include <cstdio>
#include <iostream>
#include <map>
#include <sstream>
#include <string>
#include <vector>

#include "../include/invattn.h"
#include "../invariant_attention_amd/csrc/errors.hpp"

namespace {
thread_local char g_err[512] = "";
}

ia_status ia::fail(ia_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

ia_status ia::ok() {
  g_err[0] = '\0';
  return IA_OK;
}

extern "C" const char* ia_last_error(void) { return g_err; }

int main() {
  ia_pool* pool = nullptr;
  int32_t num_pages = 0, page_size = 0;
  std::map<int, ia_seq*> seqs;
  std::string line;
  auto read_ints = [](std::istringstream& in, int n) {
    std::vector<int64_t> v((size_t)n);
    for (int i = 0; i < n; ++i) in >> v[(size_t)i];
    return v;
  };
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string op;
    if (!(in >> op)) continue;
    std::ostringstream out;
    out << op;
    if (op == "create") {
      int f;
      in >> num_pages >> page_size >> f;
      out << ' ' << ia_pool_create(num_pages, page_size, f, &pool);
    } else if (op == "begin" || op == "append") {
      int id, n;
      in >> id >> n;
      std::vector<int32_t> toks;
      for (int64_t t : read_ints(in, n)) toks.push_back((int32_t)t);
      if (op == "begin") {
        ia_seq* s = nullptr;
        int32_t cached = -1;
        const ia_status st = ia_seq_begin(pool, toks.data(), n, &s, &cached);
        if (st == IA_OK) seqs[id] = s;
        out << ' ' << st << ' ' << (st == IA_OK ? cached : 0);
      } else {
        out << ' ' << ia_seq_append_tokens(pool, seqs.at(id), toks.data(), n);
      }
    } else if (op == "reserve") {
      int id, n;
      in >> id >> n;
      std::vector<int64_t> slots((size_t)(n > 0 ? n : 1));
      const ia_status st = ia_seq_reserve(pool, seqs.at(id), n, slots.data());
      out << ' ' << st;
      if (st == IA_OK)
        for (int i = 0; i < n; ++i) out << ' ' << slots[(size_t)i];
    } else if (op == "commit") {
      int id, n;
      in >> id >> n;
      out << ' ' << ia_seq_commit(pool, seqs.at(id), n);
    } else if (op == "bt") {
      int id;
      in >> id;
      int32_t np = 0;
      ia_seq_block_table(seqs.at(id), nullptr, 0, &np);
      std::vector<int32_t> pages((size_t)(np > 0 ? np : 1));
      const ia_status st = ia_seq_block_table(seqs.at(id), pages.data(), np, &np);
      out << ' ' << st;
      for (int i = 0; i < np; ++i) out << ' ' << pages[(size_t)i];
    } else if (op == "len") {
      int id;
      in >> id;
      out << ' ' << ia_seq_len(seqs.at(id));
    } else if (op == "end") {
      int id;
      in >> id;
      out << ' ' << ia_seq_end(pool, seqs.at(id));
      seqs.erase(id);
    } else if (op == "evict") {
      int want;
      in >> want;
      int32_t ev = -1;
      const ia_status st = ia_pool_evict(pool, want, &ev);
      out << ' ' << st << ' ' << ev;
    } else if (op == "pages") {
      out << ' ' << ia_pool_num_free(pool);
      for (int32_t pg = 0; pg < num_pages; ++pg)
        out << ' ' << ia_pool_page_refs(pool, pg) << ':' << ia_pool_page_published(pool, pg);
    } else if (op == "vslots") {
      int n;
      in >> n;
      const std::vector<int64_t> s = read_ints(in, n);
      out << ' ' << ia_validate_slots(pool, s.data(), n, num_pages, page_size);
    } else {
      std::cerr << "unknown op " << op << "\n";
      return 2;
    }
    std::cout << out.str() << "\n";
  }
  for (auto& kv : seqs) ia_seq_end(pool, kv.second);
  ia_pool_destroy(pool);
  return 0;
}
